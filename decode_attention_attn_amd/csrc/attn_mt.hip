// Shared-KV decode attention with several new query tokens per sequence
// (multi-token decode: speculative or multi-token-prediction verification;
// Step-3 paper summary, "Key claims": the pages' throughput figures are
// quoted without multi-token prediction).
//
// Token T of the nt new tokens of sequence b attends, causally, to the first
// len_b - (nt - 1 - T) keys of its sequence; the tokens share every key.
// Design: the work split, cursor, LDS ring and DMAs are those of the
// one-token kernel (attn_core.h). A launch covers the tokens t0 ..; a
// workgroup has GROUPS groups of 4 waves, and wave w of group gi owns heads
// 16w..16w+15 of the NT tokens t0 + gi*NT .. t0 + gi*NT + NT - 1 (a K
// fragment read from LDS feeds the score MFMAs of every token of the wave, a
// V^T fragment its value MFMAs). Every group reads the same ring tile, so the
// cache is fetched from memory once for all GROUPS*NT tokens of a launch.
// Only group 0 issues the tile DMAs; all waves walk the same cursor and meet
// at the same barriers. q stays in registers, loaded straight from memory at
// the start of each sequence's piece. The accumulators may live in the
// accumulation registers (measured: no faster with them forced into VGPRs).
// launch_attn_mt below says which shapes are launched.
#include "attn_core.h"

namespace mfa {

// q of head 16w + n for tokens tb .. tb + NT - 1 of sequence b.
template <bool FP8, int NT>
__device__ __forceinline__ void load_q_tokens(const AttnArgs& a, int b, int tb, int w, int n, int g,
                                              bf16x8 (&qf)[NT][8]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) load_q<FP8>(a, (long long)b * a.nt + tb + t, w, n, g, qf[t]);
}

// One 32-row bf16 tile for NT tokens: each K fragment, read once, feeds the
// score products of every token; after every token's softmax step each V^T
// fragment, read once, feeds every token's value product. Fragments are
// streamed (read where they are used) so that only q, the accumulators and
// the scores stay live. nv[t] rows are valid for token t (<= 0: the token
// sees none of them and is left as it is).
template <int NT>
__device__ __forceinline__ void attend_tile_bf16_mt(const char* ks, const char* vs, const int (&nv)[NT], int n, int g,
                                                    const VReader<false>& vr, const bf16x8 (&qf)[NT][8],
                                                    float score_mul, float (&m_run)[NT], float (&l_run)[NT],
                                                    f32x4 (&acc)[NT][16]) {
  f32x4 s0[NT], s1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    s0[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    s1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bf16x8 k0 = *(const MFA_LDS bf16x8*)(ks + n * 512 + (((4 * j + g) ^ n) << 4));
    const bf16x8 k1 = *(const MFA_LDS bf16x8*)(ks + (16 + n) * 512 + (((4 * j + g) ^ n) << 4));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      s0[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[t][j], s0[t], 0, 0, 0);
      s1[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[t][j], s1[t], 0, 0, 0);
    }
  }
  bf16x8 pf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    pf[t] = nv[t] > 0 ? softmax_p(s0[t], s1[t], nv[t], g, score_mul, m_run[t], l_run[t], acc[t]) : bf16x8{};
#pragma unroll
  for (int db = 0; db < 16; ++db) {
    const bf16x8 vf = vr.read(vs, db);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[t], acc[t][db], 0, 0, 0);
  }
}

// One 64-row fp8 tile for NT tokens, 32-row block by block, streamed the same
// way: the block's K fragments feed every token's score products, each V^T
// fragment is widened once for every token's value product.
template <int NT>
__device__ __forceinline__ void attend_tile_fp8_mt(const char* ks, const char* vs, const int (&nv)[NT], int n, int g,
                                                   const VReader<true>& vr, const Q8 (&q8)[NT], float score_mul,
                                                   float (&m_run)[NT], float (&l_run)[NT], f32x4 (&acc)[NT][16]) {
  constexpr int kBlk = 32 * 256;  // bytes of a 32-row block of K or V
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    f32x4 s0[NT], s1[NT];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const i32x8 ka = read_k8(ks + blk * kBlk, n, g, 0, kk), kb = read_k8(ks + blk * kBlk, n, g, 1, kk);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        // (hi + lo / 16) as two products, the lo one scaled after
        const f32x4 la = mfma_fp8_k128(ka, q8[t].lo[kk], z), lb = mfma_fp8_k128(kb, q8[t].lo[kk], z);
        s0[t] = mfma_fp8_k128(ka, q8[t].hi[kk], kk == 0 ? z : s0[t]);
        s1[t] = mfma_fp8_k128(kb, q8[t].hi[kk], kk == 0 ? z : s1[t]);
        s0[t] += la * 0.0625f;
        s1[t] += lb * 0.0625f;
      }
    }
    bf16x8 pf[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      pf[t] = nv[t] > 32 * blk
                  ? softmax_p(s0[t], s1[t], nv[t] - 32 * blk, g, score_mul * q8[t].mul, m_run[t], l_run[t], acc[t])
                  : bf16x8{};
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const bf16x8 vf = widen8(vr.read8(vs + blk * kBlk, db));
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[t], acc[t][db], 0, 0, 0);
    }
  }
}

template <bool FP8, bool PAGED, int NT, int GROUPS>
__global__ __launch_bounds__(256 * GROUPS, 1) void attn_mt_kernel(AttnArgs a) {
  using C = Cfg<FP8>;  // the one-token ring: 4 stages of 32 KB (the q buffer is not used)
  __shared__ __attribute__((aligned(1024))) char ring[C::kStages * C::kTileBytes];
  const int lane = threadIdx.x & 63;
  const int w = uniform((int)((threadIdx.x >> 6) & 3));  // heads 16w..16w+15
  const int gi = uniform((int)(threadIdx.x >> 8));        // token group
  const int tb = a.t0 + gi * NT;                          // first token of this wave
  const int n = lane & 15;
  const int g = lane >> 4;
  const int wgi = piece_index(a.G);

  Cursor<C::kRows, PAGED> prod;
  if (!init_cursor(a, wgi, lane, prod)) return;
  Cursor<C::kRows, PAGED> cons = prod;

  // q of every token straight into registers; its loads are waited for right
  // away (before any DMA), so no later wait count has to account for them
  bf16x8 qf[NT][8];
  Q8 q8[NT];
  load_q_tokens<FP8, NT>(a, cons.b, tb, w, n, g, qf);
  wait_vmcnt<0>();
  if constexpr (FP8) {
#pragma unroll
    for (int t = 0; t < NT; ++t) split_q8(qf[t], q8[t]);
  }
  int issued = 0;
#pragma unroll
  for (int s = 0; s < C::kStages - 1; ++s) {
    if (prod.valid()) {
      if (gi == 0) issue_tile<FP8, PAGED>(a, prod, ring + s * C::kTileBytes, w, lane);
      prod.advance(a.seq_len, a.seq_off);
      ++issued;
    }
  }

  f32x4 acc[NT][16];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int db = 0; db < 16; ++db) acc[t][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
  }
  const VReader<FP8> vr(n, g);
  long long piece_lo = cons.gpos - cons.seq_start;
  bool fresh = false;
  bool drained = false;  // stores were issued since the last wait: drain fully

  for (int it = 0; cons.valid(); ++it) {
    if (fresh) {
      // a later sequence of this piece: its q (a full drain, rare)
      load_q_tokens<FP8, NT>(a, cons.b, tb, w, n, g, qf);
      wait_vmcnt<0>();
      if constexpr (FP8) {
#pragma unroll
        for (int t = 0; t < NT; ++t) split_q8(qf[t], q8[t]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        m_run[t] = -INFINITY;  // the first block rescales acc by exp2(-inf) = 0
        l_run[t] = 0.f;        // (a token that sees no row never rescales)
      }
      piece_lo = cons.gpos - cons.seq_start;
      fresh = false;
    }
    // tile `it` has landed once at most the later tiles are in flight
    wait_tiles<C::kDmaPerWave>(drained ? 0 : issued - it - 1);
    drained = false;
    __builtin_amdgcn_s_barrier();
    if (prod.valid()) {
      if (gi == 0)
        issue_tile<FP8, PAGED>(a, prod, ring + ((it + C::kStages - 1) % C::kStages) * C::kTileBytes, w, lane);
      prod.advance(a.seq_len, a.seq_off);
      ++issued;
    }
    char* stage = ring + (it % C::kStages) * C::kTileBytes;
    long long lo, hi;
    cons.tile(lo, hi);
    const int nvalid = cons.valid_rows(lo, hi);
    int nv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // causal among the new tokens: token T sees the keys before len - (nt - 1 - T)
      const long long lim = cons.len - (a.nt - 1 - (tb + t));
      const long long e = hi < lim ? hi : lim;
      nv[t] = (int)(e - lo) < nvalid ? (int)(e - lo) : nvalid;
    }
    if constexpr (FP8)
      attend_tile_fp8_mt<NT>(stage, stage + C::kHalfBytes, nv, n, g, vr, q8, a.score_mul, m_run, l_run, acc);
    else
      attend_tile_bf16_mt<NT>(stage, stage + C::kHalfBytes, nv, n, g, vr, qf, a.score_mul, m_run, l_run, acc);

    const long long pe = cons.part_end() - cons.seq_start;
    if (hi == pe) {
      // finalize this piece of sequence cons.b for every token
      const int h = 16 * w + n;
      const long long L = cons.seq_end - cons.seq_start;
      if (piece_lo == 0 && threadIdx.x == 0) {
        // this workgroup holds the sequence's first piece: tell the combine
        // where its pieces are (none when it is whole here)
        const int np = hi == L ? 0 : (int)((cons.seq_start + L - 1) / cons.per - wgi + 1);
        *(i32x2*)(a.meta + 2 * cons.b) = i32x2{wgi + cons.b, np};
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float lt = sum_over_rows(l_run[t]);
        float inv = a.v_mul / lt;
        float lse2 = m_run[t] + fast_log2(lt);
        if (!(lt > 0.f)) {  // the token saw no row of this piece: weight 0 in the merge
          inv = 0.f;
          lse2 = -INFINITY;
        }
        const long long bt = (long long)cons.b * a.nt + tb + t;  // output row of (sequence, token)
        if (piece_lo == 0 && hi == L) {
          bf16* orow = (bf16*)a.out + (bt * kHeads + h) * kHeadDim + 4 * g;
#pragma unroll
          for (int db = 0; db < 16; ++db) {
            const bf16x4 o = {(bf16)(acc[t][db][0] * inv), (bf16)(acc[t][db][1] * inv),
                              (bf16)(acc[t][db][2] * inv), (bf16)(acc[t][db][3] * inv)};
            *(bf16x4*)(orow + 16 * db) = o;
          }
          if (a.lse != nullptr && g == 0) a.lse[bt * kHeads + h] = lse2 * kLn2;
        } else {
          const long long slot = ((long long)wgi + cons.b) * a.nt + tb + t;
          bf16x8* prow = (bf16x8*)a.part_o + slot * (kHeads * kHeadDim / 8);
#pragma unroll
          for (int dp = 0; dp < 8; ++dp) {
            const f32x4 v0 = acc[t][2 * dp] * inv, v1 = acc[t][2 * dp + 1] * inv;
            prow[(w * 8 + dp) * 64 + lane] = bf16x8{(bf16)v0[0], (bf16)v0[1], (bf16)v0[2], (bf16)v0[3],
                                                    (bf16)v1[0], (bf16)v1[1], (bf16)v1[2], (bf16)v1[3]};
          }
          if (g == 0) a.part_lse[slot * kHeads + h] = lse2;
        }
      }
      fresh = true;
      drained = true;
    }
    cons.advance(a.seq_len, a.seq_off);
  }
}

template <int NT, int GROUPS>
hipError_t launch_mt(const AttnArgs& a, bool fp8, bool paged, hipStream_t stream) {
  const dim3 grid(a.G), block(256 * GROUPS);
  if (fp8)
    return paged ? launch(attn_mt_kernel<true, true, NT, GROUPS>, grid, block, stream, a)
                 : launch(attn_mt_kernel<true, false, NT, GROUPS>, grid, block, stream, a);
  return paged ? launch(attn_mt_kernel<false, true, NT, GROUPS>, grid, block, stream, a)
               : launch(attn_mt_kernel<false, false, NT, GROUPS>, grid, block, stream, a);
}

// Launch shapes: one token per wave, two groups of 4 waves per workgroup
// (two waves per SIMD hide each other's softmax and MFMA latencies; one wave
// holding two tokens, measured at 2 tokens, bf16 4K: 56 us against 46 us).
// nt = 2: one launch; nt = 3 and 4: tokens {0, 1}, then the rest in a second
// launch over the same work split (three or four groups would leave a wave
// 168 or 128 registers and spill); each launch writes its own tokens'
// outputs and partial slots, and both write the same merge records.
hipError_t launch_attn_mt(const AttnArgs& a, bool fp8, bool paged, hipStream_t stream) {
  if (a.t0 != 0 || a.nt < 2 || a.nt > 4) return hipErrorInvalidValue;
  hipError_t e = launch_mt<1, 2>(a, fp8, paged, stream);
  if (e != hipSuccess || a.nt == 2) return e;
  AttnArgs rest = a;
  rest.t0 = 2;
  return a.nt == 3 ? launch_mt<1, 1>(rest, fp8, paged, stream) : launch_mt<1, 2>(rest, fp8, paged, stream);
}

}  // namespace mfa
