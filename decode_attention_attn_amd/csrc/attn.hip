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
  void* part_o;     // [G + B][64][256] normalized partial outputs (bf16 for the MFMA kernels, fp32 otherwise)
  float* part_lse;  // [G + B][64] fp32, base-2 log-sum-exp of each partial
  int* meta;        // [B][2]: first partial slot and piece count of each sequence (0 pieces: written directly)
  const int32_t* table;  // paged cache: [B][max_blocks] page of each page-sized block (null: contiguous)
  int max_blocks;
  int page_shift;        // page = 2^page_shift rows
  int nt;                // new query tokens per sequence (1 or 2)
  int B;
  int G;
  float score_mul;  // softmax_scale * k_scale * log2(e)
  float v_mul;      // v_scale
};

constexpr int kPieceAlign = 64;  // piece lengths are multiples of this many rows

// ---------------------------------------------------------------------------
// Work split shared by the attention kernels and the combine kernel. Every
// wave computes it redundantly from seq_len (B small), so no inter-wave sync.
__device__ __forceinline__ long long piece_len(long long total, int G) {
  long long per = (total + G - 1) / G;
  return (per + kPieceAlign - 1) / kPieceAlign * kPieceAlign;
}

// Which piece a workgroup takes. Workgroups are dealt round-robin to the 8
// XCDs (workgroup i runs on XCD i % 8), so piece (i % 8) * (G / 8) + i / 8
// gives each XCD a contiguous run of pieces: the pieces of a sequence share
// one L2, so its q is fetched from memory once per XCD rather than once per
// piece, and neighbouring pieces finish together. Placement only affects
// speed; any bijection of the workgroup indices is correct.
__device__ __forceinline__ int piece_index(int G) {
  const int i = blockIdx.x;
  return (G & 7) == 0 ? (i & 7) * (G >> 3) + (i >> 3) : i;
}

// A sequence's length in the work split. A paged cache pads every sequence
// to a whole number of tiles, so that tiles (multiples of kRows from the
// sequence's first row) never straddle a page; the padding rows are masked.
template <int kRows, bool PAGED>
__device__ __forceinline__ long long split_len(long long len) {
  return PAGED ? (len + kRows - 1) / kRows * kRows : len;
}

// Walks one workgroup's piece tile by tile (wave-uniform state).
template <int kRows, bool PAGED = false>
struct Cursor {
  long long gpos, r1;            // next global position, end of the workgroup's piece
  long long per;                 // piece length (rows per workgroup)
  long long seq_start, seq_end;  // global range of the current sequence
  long long off;                 // cache row of the sequence's first key (contiguous cache)
  long long len;                 // the sequence's length (seq_end - seq_start less the paging pad)
  int b;

  __device__ __forceinline__ bool valid() const { return gpos < r1; }
  __device__ __forceinline__ long long part_end() const { return seq_end < r1 ? seq_end : r1; }
  // Rows [lo, hi) of the current tile, relative to the sequence start.
  __device__ __forceinline__ void tile(long long& lo, long long& hi) const {
    lo = gpos - seq_start;
    const long long e = gpos + kRows;
    const long long pe = part_end();
    hi = (e < pe ? e : pe) - seq_start;
  }
  __device__ __forceinline__ void advance(const int32_t* len, const int64_t* offs) {
    const long long pe = part_end();
    const long long e = gpos + kRows;
    gpos = e < pe ? e : pe;
    if (gpos == seq_end && gpos < r1) {
      long long n;
      do {
        ++b;
        seq_start = seq_end;
        n = load_scalar(len, b);
        seq_end = seq_start + split_len<kRows, PAGED>(n);
      } while (seq_end == seq_start);
      this->len = n;
      if (!PAGED) off = load_scalar(offs, b);
    }
  }
  // rows of the current tile that hold keys
  __device__ __forceinline__ int valid_rows(long long lo, long long hi) const {
    return (int)((PAGED && hi > len ? len : hi) - lo);
  }
};

// A workgroup's start: total length, piece length, and the sequence holding
// its first position r0 = wgi * per (with that sequence's start and cache
// offset). Kept short: it runs before the first tile load, when the code is
// not yet in the instruction cache and every fetch of it queues behind the
// tile loads of the workgroups that got going first. The first 64 sequences
// stay in registers; more are re-read chunk by chunk.
template <int kRows, bool PAGED>
__device__ __forceinline__ bool init_cursor(const AttnArgs& a, int wgi, int lane, Cursor<kRows, PAGED>& c) {
  const int B = a.B;
  const int ic = lane < B ? lane : B - 1;
  const long long n0 = lane < B ? (long long)a.seq_len[ic] : 0;
  const long long v0 = split_len<kRows, PAGED>(n0);
  const long long o0 = PAGED ? 0 : a.seq_off[ic];
  long long sum = v0;
  for (int i = 64 + lane; i < B; i += 64) sum += split_len<kRows, PAGED>(a.seq_len[i]);
  const long long total = uniform(wave_sum_ll(sum));
  const long long per = piece_len(total, a.G);
  const long long r0 = (long long)wgi * per;
  if (r0 >= total) return false;
  long long base = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int i = c0 + lane;
    const long long n = c0 == 0 ? n0 : (i < B ? (long long)a.seq_len[i] : 0);
    const long long v = split_len<kRows, PAGED>(n);
    long long incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const long long t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    const unsigned long long hit = __ballot(i < B && base + incl > r0);
    if (hit) {
      const int first = __ffsll((long long)hit) - 1;
      const int b = uniform(c0 + first);
      const long long start = uniform(base + __shfl(incl - v, first));
      c.r1 = r0 + per < total ? r0 + per : total;
      c.per = per;
      c.gpos = r0;
      c.b = b;
      c.seq_start = start;
      c.seq_end = start + uniform(__shfl(v, first));
      c.len = uniform(__shfl(n, first));
      c.off = PAGED ? 0 : (c0 == 0 ? uniform(__shfl(o0, first)) : load_scalar(a.seq_off, b));
      return true;
    }
    base += __shfl(incl, 63);
  }
  return false;  // not reached: r0 < total
}

// ---------------------------------------------------------------------------
// MFMA kernel (bf16 q; bf16 or fp8 cache).
// NT = new query tokens per sequence (1, or 2 for multi-token decode): wave w
// serves token w / 4, heads 16 (w % 4)..+15, so NT tokens take 4 NT waves,
// and their q (32 KB each) sit beside the ring.
template <bool FP8, int NT = 1>
struct Cfg {
  static constexpr int kRowBytes = FP8 ? 256 : 512;
  static constexpr int kRows = FP8 ? 64 : 32;                     // cache rows per tile
  static constexpr int kHalfBytes = kRows * kRowBytes;             // K (or V) part of a tile: 16 KB
  static constexpr int kTileBytes = 2 * kHalfBytes;                // 32 KB
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kRowsPerBlock = 1024 / kRowBytes;           // rows per 1 KB DMA block
  static constexpr int kWaves = 4 * NT;
  static constexpr int kBlocksPerWave = kHalfBytes / 1024 / kWaves;  // DMA blocks per wave per half: 4 (2)
  static constexpr int kDmaPerWave = 2 * kBlocksPerWave;             // DMA instructions per wave per tile: 8 (4)
  static constexpr int kStages = NT == 1 ? 4 : 3;                    // LDS ring: 3 (2) tiles in flight
  static constexpr int kSteadyVm = (kStages - 2) * kDmaPerWave;      // DMAs still in flight once a tile landed
  static constexpr int kLdsBytes = kStages * kTileBytes + NT * kHeads * kHeadDim * 2;  // 160 KB
};

// XOR swizzles of 16-byte chunks within a row (row r = 0..31 of a 32-row block).
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v16(int r) { return (r & 7) << 1; }
__device__ __forceinline__ int swz_v8(int r) { return (r & 3) | (((r >> 4) & 1) << 2) | (((r >> 2) & 1) << 3); }

// Cache policy of the K/V tile DMAs: nontemporal (each cache byte is read
// once per call). Measured on MI355X against the default policy: bf16 4K
// 33.6 -> 33.1 us, fp8 4K -1 %, the 8K-64K ragged batch 123 -> 115 us.
constexpr int kCpolNT = 2;

// Direct-to-LDS DMA of the producer's current tile into a ring stage. Lane i of
// a wave moves 16 bytes into LDS slot i of a 1 KB block, so the XOR swizzle is
// applied on the global side: slot (row r, chunk pc) receives global chunk
// pc ^ swz(r). Each row is still read as one full run. Rows past the valid
// end re-read the last valid row (their scores are masked to -inf).
template <bool FP8, bool PAGED, int NT>
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const Cursor<Cfg<FP8>::kRows, PAGED>& c, char* stage,
                                           int w, int lane) {
  using C = Cfg<FP8, NT>;
  long long lo, hi;
  c.tile(lo, hi);
  long long row0;  // cache row of the tile's first key
  if constexpr (PAGED) {
    // the tile lies inside one page (tiles start at multiples of kRows, a
    // page holds a whole number of tiles): one table entry per tile
    const long long page = load_scalar(a.table, (long long)c.b * a.max_blocks + (lo >> a.page_shift));
    row0 = (page << a.page_shift) + (lo & ((1LL << a.page_shift) - 1));
  } else {
    row0 = c.off + lo;
  }
  const char* kb = (const char*)a.k + row0 * C::kRowBytes;
  const char* vb = (const char*)a.v + row0 * C::kRowBytes;
  const int nvalid = c.valid_rows(lo, hi);
  const int r_in = lane / C::kChunksPerRow;
  const int pc = lane % C::kChunksPerRow;
#pragma unroll
  for (int jj = 0; jj < C::kBlocksPerWave; ++jj) {
    const int blk = w * C::kBlocksPerWave + jj;
    const int r = blk * C::kRowsPerBlock + r_in;
    const int rr = r < nvalid ? r : nvalid - 1;
    const int r32 = r & 31;
    const int ck = pc ^ swz_k(r32);
    const int cv = pc ^ (FP8 ? swz_v8(r32) : swz_v16(r32));
    __builtin_amdgcn_global_load_lds((const void*)(kb + (long long)rr * C::kRowBytes + ck * 16),
                                     (MFA_LDS void*)(stage + blk * 1024), 16, 0, kCpolNT);
    __builtin_amdgcn_global_load_lds((const void*)(vb + (long long)rr * C::kRowBytes + cv * 16),
                                     (MFA_LDS void*)(stage + C::kHalfBytes + blk * 1024), 16, 0, kCpolNT);
  }
}

// q of sequence b ([64 heads][256] bf16, 32 KB) goes HBM -> LDS by DMA like
// the cache tiles: it is then tracked by the same wait counts, so the
// prologue can wait for q and the first tile only, and the compiler never
// sees q as a pending register load.
// With NT tokens the NT q blocks of a sequence are contiguous ([B][NT][64][256]).
template <int NT>
__device__ __forceinline__ void issue_q(const AttnArgs& a, int b, char* qs, int w, int lane) {
  const char* src = (const char*)a.q + (long long)b * NT * (kHeads * kHeadDim * 2);
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int blk = w * 8 + jj;  // 32 NT blocks of 1 KB, 8 per wave
    __builtin_amdgcn_global_load_lds((const void*)(src + blk * 1024 + lane * 16), (MFA_LDS void*)(qs + blk * 1024),
                                     16, 0, 0);
  }
}

// q of head 16w + n, the channels this lane's k-slot group g supplies to the
// score product: bf16 step j covers channels 32j + 8g..+7; fp8 step kk (k = 128)
// covers channels 128kk + 32g..+31 (qf[4kk + m] holds 128kk + 32g + 8m..+7).
template <bool FP8>
__device__ __forceinline__ void read_q(const char* qs, int w, int n, int g, bf16x8 (&qf)[8]) {
  const char* row = qs + (16 * w + n) * (kHeadDim * 2);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d0 = FP8 ? (128 * (j >> 2) + 32 * g + 8 * (j & 3)) : (32 * j + 8 * g);
    qf[j] = lds_read_b128((const MFA_LDS bf16x8*)(row + 2 * d0));
  }
}

// ---------------------------------------------------------------------------
// fp8 cache, score product: the cache's K bytes feed the gfx950 fp8 MFMA
// (v_mfma_f32_16x16x128_f8f6f4, e4m3 operands, twice the bf16 rate) without
// any widening. q is carried as two e4m3 numbers, q ~ 2^e (hi + lo / 16) with
// hi = fp8(q 2^-e) and lo = fp8(16 (q 2^-e - hi)), where 2^e puts the head's
// largest |q| in [128, 256); the pair keeps about 8 significant bits (as bf16
// does) and two k = 128 fp8 products cost what one bf16 product of the same
// width does. (A single fp8 q would keep 4 bits.)
struct Q8 {
  i32x8 hi[2], lo[2];  // score step kk: channels 128kk + 32g..+31, byte i <-> channel 128kk + 32g + i
  float mul;           // 2^e
};

// 32 floats -> 32 e4m3 bytes (round to nearest even), byte i <- v[i].
__device__ __forceinline__ i32x8 pack_fp8x32(const float (&v)[32]) {
  i32x8 r;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * d], v[4 * d + 1], 0, false);
    r[d] = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * d + 2], v[4 * d + 3], x, true);
  }
  return r;
}

__device__ __forceinline__ void split_q8(const bf16x8 (&qf)[8], Q8& q) {
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf((float)qf[j][i]));
  mx = max_over_rows(mx);  // the 4 lanes of a head hold all its channels
  int e = 0;
  if (mx > 0.f) {
    int ex;
    frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
    e = ex - 8;
  }
  q.mul = ldexpf(1.f, e);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    float v[32], r[32];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 8; ++i) v[8 * m + i] = ldexpf((float)qf[4 * kk + m][i], -e);
    q.hi[kk] = pack_fp8x32(v);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const f32x2 b0 = __builtin_amdgcn_cvt_pk_f32_fp8(q.hi[kk][d], false);
      const f32x2 b1 = __builtin_amdgcn_cvt_pk_f32_fp8(q.hi[kk][d], true);
      r[4 * d] = (v[4 * d] - b0[0]) * 16.f;
      r[4 * d + 1] = (v[4 * d + 1] - b0[1]) * 16.f;
      r[4 * d + 2] = (v[4 * d + 2] - b1[0]) * 16.f;
      r[4 * d + 3] = (v[4 * d + 3] - b1[1]) * 16.f;
    }
    q.lo[kk] = pack_fp8x32(r);
  }
}

// fp8 K operand of score step kk for rows 16pb..16pb+15 of the 32-row block
// at ks: row 16pb + n, channels 128kk + 32g..+31 = chunks 8kk + 2g and
// 8kk + 2g + 1, stored at slots chunk ^ n.
__device__ __forceinline__ i32x8 read_k8(const char* ks, int n, int g, int pb, int kk) {
  const char* row = ks + (16 * pb + n) * 256;
  const int c = 8 * kk + 2 * g;
  const u32x4 a = *(const MFA_LDS u32x4*)(row + ((c ^ n) << 4));
  const u32x4 b = *(const MFA_LDS u32x4*)(row + (((c + 1) ^ n) << 4));
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ f32x4 mfma_fp8_k128(const i32x8& a, const i32x8& b, const f32x4& c) {
  // e4m3 x e4m3 (format code 0), unit scales
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// bf16 K operand (A of S^T = K Q^T) for rows 16pb..16pb+15 of the 32-row
// block at ks: kf[j] holds the 8 channels of k-slot group g at step j for row
// 16pb + n. (The fp8 score product reads K with read_k8.)
__device__ __forceinline__ void read_k(const char* ks, int n, int g, bf16x8 (&kf)[8], int pb) {
#pragma unroll
  for (int j = 0; j < 8; ++j) kf[j] = *(const MFA_LDS bf16x8*)(ks + (16 * pb + n) * 512 + (((4 * j + g) ^ n) << 4));
}

// V^T operand (A of O^T = V^T P^T): the fragment of channel block db holds,
// for channel 16db + n, the cache rows of k-slots 8g..8g+7, i.e. rows
// 16b + 4g + i (b = 0,1; i = 0..3) of the 32-row block.
template <bool FP8>
struct VReader {
  int base0, base1, sw0, sw1, lc_lo;  // bf16 (tr16: two reads of 4 rows)
  int base, sw;                       // fp8 (tr8: one read of 8 rows)
  __device__ __forceinline__ VReader(int n, int g) {
    if constexpr (!FP8) {
      // lane i of a 16-lane group supplies row 4g + i/4 (+16), channels 4(i%4)..+3
      const int rq = n >> 2;
      const int half = (n & 1) << 3;
      lc_lo = (n & 3) >> 1;
      const int r0 = 4 * g + rq, r1 = 16 + 4 * g + rq;
      base0 = r0 * 512 + half;
      base1 = r1 * 512 + half;
      sw0 = swz_v16(r0);
      sw1 = swz_v16(r1);
    } else {
      // lane i of a 16-lane group supplies k-slot row r' = i/2, byte half i&1
      const int rp = n >> 1;
      const int r = 16 * (rp >> 2) + 4 * g + (rp & 3);
      base = r * 256 + ((n & 1) << 3);
      sw = swz_v8(r);
    }
  }
  // fp8: the 8 raw bytes of the fragment (widened with widen8)
  __device__ __forceinline__ i32x2 read8(const char* vs, int db) const {
    static_assert(FP8, "bf16 fragments are read with read");
    return lds_read_tr8((const MFA_LDS i32x2*)(vs + base + ((db ^ sw) << 4)));
  }
  // bf16: the fragment
  __device__ __forceinline__ bf16x8 read(const char* vs, int db) const {
    static_assert(!FP8, "fp8 fragments are read with read8");
    const int lc = 2 * db + lc_lo;
    const bf16x4 lo = lds_read_tr16((const MFA_LDS bf16x4*)(vs + base0 + ((lc ^ sw0) << 4)));
    const bf16x4 hi = lds_read_tr16((const MFA_LDS bf16x4*)(vs + base1 + ((lc ^ sw1) << 4)));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

__device__ __forceinline__ bf16x8 widen8(const i32x2& raw) {
  bf16x8 v;
  fp8x4_to_bf16((unsigned)raw[0], v, 0);
  fp8x4_to_bf16((unsigned)raw[1], v, 4);
  return v;
}

// Online-softmax update and value product of one 32-row block whose scores
// (before score_mul) are s0 (rows 4g+i) and s1 (rows 16+4g+i) of head n; vf
// holds the block's V^T operands. Rows at or past nvalid are masked (a block
// with none left changes nothing once m_run is finite).
__device__ __forceinline__ void softmax_pv(const f32x4& s0, const f32x4& s1, int nvalid, int g, float score_mul,
                                           const bf16x8 (&vf)[16], float& m_run, float& l_run, f32x4 (&acc)[16]) {
  float sc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = (4 * g + i < nvalid) ? s0[i] * score_mul : -INFINITY;
    sc[4 + i] = (16 + 4 * g + i < nvalid) ? s1[i] * score_mul : -INFINITY;
  }
  float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
  mx = max_over_rows(mx);
  // Lazy rescale: the reference max only moves when a score exceeds it by
  // more than 8 (base 2), so exponentials stay <= 256 (no bf16/fp32 range
  // issue) and the O rescale runs on a piece's first block and rarely after.
  const bool jump = mx > m_run + 8.f;
  if (__ballot(jump)) {
    const float m_new = jump ? mx : m_run;
    const float alpha = fast_exp2(m_run - m_new);  // 0 on a fresh piece (m_run = -inf)
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 16; ++db) acc[db] *= alpha;
    m_run = m_new;
  }
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = fast_exp2(sc[i] - m_run);
    l_run += p[i];
  }
  const bf16x8 pf = {(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3], (bf16)p[4], (bf16)p[5], (bf16)p[6], (bf16)p[7]};
#pragma unroll
  for (int db = 0; db < 16; ++db) acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pf, acc[db], 0, 0, 0);
}

// One 32-row bf16 tile: scores, online softmax update, PV accumulate. The K
// fragments are read first, then the score MFMAs are interleaved with the V
// reads (V does not depend on the scores), so that LDS latency overlaps
// matrix work.
__device__ __forceinline__ void attend_tile_bf16(const char* ks, const char* vs, int nvalid, int n, int g,
                                                 const VReader<false>& vr, const bf16x8 (&qf)[8], float score_mul,
                                                 float& m_run, float& l_run, f32x4 (&acc)[16]) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  bf16x8 vf[16];
  bf16x8 kf0[8], kf1[8];
  read_k(ks, n, g, kf0, 0);
  read_k(ks, n, g, kf1, 1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf0[j], qf[j], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf1[j], qf[j], s1, 0, 0, 0);
    vf[2 * j] = vr.read(vs, 2 * j);
    vf[2 * j + 1] = vr.read(vs, 2 * j + 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  softmax_pv(s0, s1, nvalid, g, score_mul, vf, m_run, l_run, acc);
}

// Scores of the fp8 32-row block at ks, before score_mul: rows 4g+i (s0) and
// 16+4g+i (s1) of head n, as hi + lo / 16 products.
__device__ __forceinline__ void scores_fp8(const char* ks, int n, int g, const Q8& q8, f32x4& s0, f32x4& s1) {
  const i32x8 k00 = read_k8(ks, n, g, 0, 0), k01 = read_k8(ks, n, g, 0, 1);
  const i32x8 k10 = read_k8(ks, n, g, 1, 0), k11 = read_k8(ks, n, g, 1, 1);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 l0 = mfma_fp8_k128(k00, q8.lo[0], z);
  f32x4 l1 = mfma_fp8_k128(k10, q8.lo[0], z);
  s0 = mfma_fp8_k128(k00, q8.hi[0], z);
  s1 = mfma_fp8_k128(k10, q8.hi[0], z);
  l0 = mfma_fp8_k128(k01, q8.lo[1], l0);
  l1 = mfma_fp8_k128(k11, q8.lo[1], l1);
  s0 = mfma_fp8_k128(k01, q8.hi[1], s0);
  s1 = mfma_fp8_k128(k11, q8.hi[1], s1);
  s0 += l0 * 0.0625f;
  s1 += l1 * 0.0625f;
}

// One 64-row fp8 tile as two 32-row blocks, ordered so that matrix and vector
// work of the two blocks overlap within the wave: both blocks' score products
// are issued before the first block's softmax (which then runs on the vector
// unit while the second block's products execute), and the second block's
// softmax and V widening follow the issue of the first block's value product.
// kEarlyV: read the second block's V with the first's (one wave per SIMD has
// the registers; with two waves per SIMD it is read after the first softmax).
template <bool kEarlyV>
__device__ __forceinline__ void attend_tile_fp8(const char* ks, const char* vs, int nvalid, int n, int g,
                                                const VReader<true>& vr, const Q8& q8, float score_mul, float& m_run,
                                                float& l_run, f32x4 (&acc)[16]) {
  constexpr int kBlk = 32 * 256;  // bytes of a 32-row block of K or V
  score_mul *= q8.mul;
  f32x4 a0, a1, b0, b1;
  i32x2 v8[16], w8[kEarlyV ? 16 : 1];
  bf16x8 vf[16];
  scores_fp8(ks, n, g, q8, a0, a1);
#pragma unroll
  for (int db = 0; db < 16; ++db) v8[db] = vr.read8(vs, db);
  // rows past nvalid are masked, so the second block needs no branch
  scores_fp8(ks + kBlk, n, g, q8, b0, b1);
  if constexpr (kEarlyV) {
#pragma unroll
    for (int db = 0; db < 16; ++db) w8[db] = vr.read8(vs + kBlk, db);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int db = 0; db < 16; ++db) vf[db] = widen8(v8[db]);
  softmax_pv(a0, a1, nvalid, g, score_mul, vf, m_run, l_run, acc);
  if constexpr (!kEarlyV) {
#pragma unroll
    for (int db = 0; db < 16; ++db) v8[db] = vr.read8(vs + kBlk, db);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int db = 0; db < 16; ++db) {
    if constexpr (kEarlyV)
      vf[db] = widen8(w8[db]);
    else
      vf[db] = widen8(v8[db]);
  }
  softmax_pv(b0, b1, nvalid - 32, g, score_mul, vf, m_run, l_run, acc);
}

template <bool FP8, bool PAGED, int NT>
__global__ __launch_bounds__(256 * NT, 1) void attn_mfma_kernel(AttnArgs a) {
  using C = Cfg<FP8, NT>;
  // the tile ring, then q (32 KB per token): 160 KB of LDS
  __shared__ __attribute__((aligned(1024))) char ring[C::kLdsBytes];
  char* const qs = ring + C::kStages * C::kTileBytes;
  const int lane = threadIdx.x & 63;
  const int wv = uniform((int)(threadIdx.x >> 6));
  const int w = wv & 3;    // heads 16w..16w+15
  const int tok = wv >> 2;  // new token (multi-token decode; 0 otherwise)
  char* const qt = qs + tok * (kHeads * kHeadDim * 2);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int wgi = piece_index(a.G);

  Cursor<C::kRows, PAGED> prod;
  if (!init_cursor(a, wgi, lane, prod)) return;
  Cursor<C::kRows, PAGED> cons = prod;

  // q of the first piece goes out ahead of the first tile DMAs.
  issue_q<NT>(a, cons.b, qs, wv, lane);
  int issued = 0;
#pragma unroll
  for (int s = 0; s < C::kStages - 1; ++s) {
    if (prod.valid()) {
      issue_tile<FP8, PAGED, NT>(a, prod, ring + s * C::kTileBytes, wv, lane);
      prod.advance(a.seq_len, a.seq_off);
      ++issued;
    }
  }
  // q and tile 0 have landed once at most the later prologue tiles are in
  // flight (DMAs complete in issue order); the loop's first step then refills
  // right away.
  if (issued == 3)
    wait_vmcnt<2 * C::kDmaPerWave>();
  else if (issued == 2)
    wait_vmcnt<C::kDmaPerWave>();
  else
    wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  bf16x8 qf[8];
  read_q<FP8>(qt, w, n, g, qf);
  Q8 q8;  // fp8 cache: q as hi/lo e4m3 pairs
  if constexpr (FP8) split_q8(qf, q8);

  f32x4 acc[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const VReader<FP8> vr(n, g);
  float m_run = -INFINITY, l_run = 0.f;
  long long piece_lo = cons.gpos - cons.seq_start;
  bool fresh = false;
  bool drained = false;  // stores were issued since the last wait: drain fully

  for (int t = 0; cons.valid(); ++t) {
    if (fresh) {
      // Later pieces of the workgroup: a full drain for their q (rare). Every
      // wave finished reading the previous q right after it landed.
      issue_q<NT>(a, cons.b, qs, wv, lane);
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      read_q<FP8>(qt, w, n, g, qf);
      if constexpr (FP8) split_q8(qf, q8);
      m_run = -INFINITY;  // the first block rescales acc by exp2(-inf) = 0
      // (a token that sees no row of the new piece never rescales: its sum
      // must start from zero for the empty-token test at the piece's end)
      if constexpr (NT > 1) l_run = 0.f;
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
      issue_tile<FP8, PAGED, NT>(a, prod, ring + ((t + C::kStages - 1) % C::kStages) * C::kTileBytes, wv, lane);
      prod.advance(a.seq_len, a.seq_off);
      ++issued;
    }
    char* stage = ring + (t % C::kStages) * C::kTileBytes;
    long long lo, hi;
    cons.tile(lo, hi);
    int nvalid = cons.valid_rows(lo, hi);
    if constexpr (NT > 1) {
      // causal among the new tokens: token tok sees the rows before len - (NT - 1 - tok)
      const long long lim = cons.len - (NT - 1 - tok);
      nvalid = (int)((hi < lim ? hi : lim) - lo);
    }
    if (NT == 1 || nvalid > 0) {
      if constexpr (FP8)
        attend_tile_fp8<NT == 1>(stage, stage + C::kHalfBytes, nvalid, n, g, vr, q8, a.score_mul, m_run, l_run,
                                 acc);
      else
        attend_tile_bf16(stage, stage + C::kHalfBytes, nvalid, n, g, vr, qf, a.score_mul, m_run, l_run, acc);
    }

    const long long pe = cons.part_end() - cons.seq_start;
    if (hi == pe) {
      // finalize this piece of sequence cons.b (for token tok)
      const float lt = sum_over_rows(l_run);
      float inv = a.v_mul / lt;
      float lse2 = m_run + fast_log2(lt);
      if constexpr (NT > 1) {
        if (!(lt > 0.f)) {  // the token saw no row of this piece: weight 0 in the merge
          inv = 0.f;
          lse2 = -INFINITY;
        }
      }
      const int h = 16 * w + n;
      const long long bt = (long long)cons.b * NT + tok;  // output row of (sequence, token)
      const long long L = cons.seq_end - cons.seq_start;
      if (piece_lo == 0 && threadIdx.x == 0) {
        // this workgroup holds the sequence's first piece: tell the combine
        // where its pieces are (w0 = wgi; none when it is whole here)
        const int np = hi == L ? 0 : (int)((cons.seq_start + L - 1) / cons.per - wgi + 1);
        *(i32x2*)(a.meta + 2 * cons.b) = i32x2{wgi + cons.b, np};
      }
      if (piece_lo == 0 && hi == L) {
        bf16* orow = (bf16*)a.out + (bt * kHeads + h) * kHeadDim + 4 * g;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
          const bf16x4 o = {(bf16)(acc[db][0] * inv), (bf16)(acc[db][1] * inv), (bf16)(acc[db][2] * inv),
                            (bf16)(acc[db][3] * inv)};
          *(bf16x4*)(orow + 16 * db) = o;
        }
        if (a.lse != nullptr && g == 0) a.lse[bt * kHeads + h] = lse2 * kLn2;
      } else {
        // partial outputs in bf16 (half the bytes of the round trip through
        // memory; the merge weights stay fp32), in the register layout: one
        // 1 KB contiguous store per wave and channel-block pair (the combine
        // knows the map)
        const long long slot = ((long long)wgi + cons.b) * NT + tok;
        bf16x8* prow = (bf16x8*)a.part_o + slot * (kHeads * kHeadDim / 8);
#pragma unroll
        for (int dp = 0; dp < 8; ++dp) {
          const f32x4 v0 = acc[2 * dp] * inv, v1 = acc[2 * dp + 1] * inv;
          prow[(w * 8 + dp) * 64 + lane] = bf16x8{(bf16)v0[0], (bf16)v0[1], (bf16)v0[2], (bf16)v0[3],
                                                  (bf16)v1[0], (bf16)v1[1], (bf16)v1[2], (bf16)v1[3]};
        }
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
  // workgroup (bt, y): channel block y of output row bt = (sequence b, token tok)
  const int bt = blockIdx.x;
  const int nt = a.nt;  // 1, or 2 for multi-token decode
  const int b = nt == 1 ? bt : bt >> 1;
  const int tok = bt - b * nt;
  const int c = blockIdx.y * 256 + threadIdx.x;
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
  a.B = p.B;
  a.G = p.G;
  a.score_mul = p.softmax_scale * p.k_scale * kLog2e;
  a.v_mul = p.v_scale;
  const dim3 block(256);
  const dim3 comb_f32(p.B, 16);
  const dim3 comb_mfma(p.B * p.nt, 8);
  hipError_t e = hipSuccess;
  switch (p.kind) {
    case AttnKind::F32:
      e = launch(attn_f32_kernel, dim3(p.G), block, stream, a);
      if (e == hipSuccess) e = launch(attn_combine_f32_kernel, comb_f32, block, stream, a);
      break;
    case AttnKind::BF16:
      if (p.nt == 2)
        e = p.table ? launch(attn_mfma_kernel<false, true, 2>, dim3(p.G), dim3(512), stream, a)
                    : launch(attn_mfma_kernel<false, false, 2>, dim3(p.G), dim3(512), stream, a);
      else
        e = p.table ? launch(attn_mfma_kernel<false, true, 1>, dim3(p.G), block, stream, a)
                    : launch(attn_mfma_kernel<false, false, 1>, dim3(p.G), block, stream, a);
      if (e == hipSuccess) e = launch(attn_combine_mfma_kernel, comb_mfma, block, stream, a);
      break;
    case AttnKind::BF16_FP8KV:
      if (p.nt == 2)
        e = p.table ? launch(attn_mfma_kernel<true, true, 2>, dim3(p.G), dim3(512), stream, a)
                    : launch(attn_mfma_kernel<true, false, 2>, dim3(p.G), dim3(512), stream, a);
      else
        e = p.table ? launch(attn_mfma_kernel<true, true, 1>, dim3(p.G), block, stream, a)
                    : launch(attn_mfma_kernel<true, false, 1>, dim3(p.G), block, stream, a);
      if (e == hipSuccess) e = launch(attn_combine_mfma_kernel, comb_mfma, block, stream, a);
      break;
  }
  return e;
}

}  // namespace mfa
