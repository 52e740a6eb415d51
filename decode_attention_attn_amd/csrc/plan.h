// Host-side planning of the projection GEMMs and of the projection calls'
// workspace layouts. Plain arithmetic with no HIP dependency: the C ABI and
// the kernel launchers share it, and a CPU test compiles it on its own to
// check that a workspace sized without a device fits the plan made on any
// device.
#pragma once

#include <stddef.h>

namespace mfa {

constexpr int kGemmTileM = 128;    // batch rows per GEMM workgroup
constexpr int kGemmChunkK = 64;    // K per pipeline stage
constexpr int kGemmTileN = 128;    // output columns of the narrow tile (the wide one has 256)
constexpr int kPlanCus = 256;      // most compute units a plan is made for (MI355X has 256)

struct GemmPlan {
  int M, N, K, N0;
  int splits;   // S: the K dimension is cut into S parts, each adding fp32 partial sums
  int mchunks;  // ceil(M / 128) (bf16 path)
  int tile_n;   // output columns per workgroup (bf16 path): 64 or 128 for bf16
                // weights, 128 or 256 for block-fp8 weights
  bool w8;      // made for block-fp8 weights
};

// Split-K factor of a tile width on `cus` compute units: the workgroups fill
// the compute units once (a second partial wave would only lengthen the
// tail), with at least 4 K chunks per split (below that a workgroup is all
// start-up latency and the partial sums outgrow the weights).
inline int gemm_splits(int M, int N, int K, int tn, int cus) {
  const int tiles = (N / tn) * ((M + kGemmTileM - 1) / kGemmTileM);
  const int nch = K / kGemmChunkK;
  const int smax = nch / 4 > 0 ? nch / 4 : 1;
  int s = cus / tiles;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  return s;
}

// Activation bytes up to which a bf16-weight product takes 64-column tiles:
// the 64-column tile reads two activation bytes per weight byte, which costs
// nothing while the activations stay in L2 (q down-projection, K/V, q
// up-projection at batch 128); the out-projection's 4 MB of activations take
// 128-column tiles. Measured on MI355X at batch 128 (product + split-K sum):
// q up 25.6 -> 18.4 us, [W_dq; W_k; W_v] 18.7 -> 15.2 us, out-projection
// 61.5 -> 56.7 us against the block-fp8 kernel's tiling.
constexpr long long kPipeSmallX = 2LL << 20;

// bf16 weights: the tile width above and its split. Block-fp8 weights: for
// each of the 128/256-column widths the split above, then the width with the
// smaller estimated time: each CU streams (tile_n + 128) * K / S * 2 bytes of
// weights and activations (~30 GB/s per CU), and the partial sums add
// 2 * S * M * N * 4 bytes across the chip (~5 TB/s). fp32 (VALU path): one
// plain pass, no split.
inline GemmPlan plan_gemm(bool bf16_path, int M, int N, int K, int N0, int cus, bool w8 = false) {
  GemmPlan p{M, N, K, N0, 1, 1, kGemmTileN, w8};
  if (!bf16_path) return p;
  if (cus < 1) cus = 1;
  if (cus > kPlanCus) cus = kPlanCus;
  p.mchunks = (M + kGemmTileM - 1) / kGemmTileM;
  if (!w8) {
    p.tile_n = (N % 128 != 0 || (long long)M * K * 2 <= kPipeSmallX) ? 64 : 128;
    p.splits = gemm_splits(M, N, K, p.tile_n, cus);
    return p;
  }
  double best = 0.0;
  for (int tn = 128; tn <= 256; tn *= 2) {
    if (N % tn != 0) continue;
    const int tiles = (N / tn) * p.mchunks;
    const int s = gemm_splits(M, N, K, tn, cus);
    const int waves = (tiles * s + cus - 1) / cus;
    const double per_cu = (double)(tn + kGemmTileM) * K / s * 2.0 * waves;
    const double partial = s > 1 ? 2.0 * s * M * (double)N * 4.0 : 0.0;
    const double t = per_cu / 30e9 + partial / 5e12;
    if (best == 0.0 || t < best) {
      best = t;
      p.tile_n = tn;
      p.splits = s;
    }
  }
  return p;
}

inline size_t gemm_partial_bytes(const GemmPlan& p) { return (size_t)p.splits * p.M * p.N * sizeof(float); }

// Partial-sum bytes that bound every bf16 plan of this product, for either
// weight format, on 1..256 compute units: the bf16-weight width does not
// depend on the CU count and each width's split only grows with it, so the
// largest split of any width at 256 CUs bounds what any device picks.
inline size_t gemm_partial_bound(int M, int N, int K) {
  size_t best = (size_t)plan_gemm(true, M, N, K, N, kPlanCus, false).splits * M * N * sizeof(float);
  for (int tn = 128; tn <= 256; tn *= 2) {
    if (N % tn != 0) continue;
    const size_t b = (size_t)gemm_splits(M, N, K, tn, kPlanCus) * M * N * sizeof(float);
    if (b > best) best = b;
  }
  return best;
}

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Dimensions of the projections.
constexpr int kPlanHidden = 7168, kPlanRank = 2048, kPlanQDim = 16384, kPlanHeadDim = 256;

// Workspace of the q path: fp32 partial sums of the down-projection (later
// reused by the up-projection's), then the normalized latent c_hat.
struct QprojLayout {
  size_t part_bytes;  // region reserved for partial sums
  size_t chat_offset;
  size_t total;
};
inline QprojLayout qproj_layout(int B, bool bf) {
  QprojLayout l;
  if (bf) {
    const size_t dn = gemm_partial_bound(B, kPlanRank, kPlanHidden);
    const size_t up = gemm_partial_bound(B, kPlanQDim, kPlanRank);
    l.part_bytes = dn > up ? dn : up;
  } else {
    l.part_bytes = (size_t)B * kPlanRank * sizeof(float);
  }
  l.chat_offset = align256(l.part_bytes);
  l.total = l.chat_offset + align256((size_t)B * kPlanRank * (bf ? 2 : 4));
  return l;
}
// Bytes of the q path's partial sums under one device's plans.
// The q path with the K/V projections folded into its down-projection (one
// GEMM over [W_dq; W_k; W_v], bf16 only): the same layout with 2560 columns
// in the first product.
constexpr int kPlanQkv = kPlanRank + 2 * kPlanHeadDim;
inline QprojLayout qkv_layout(int B) {
  QprojLayout l;
  const size_t dn = gemm_partial_bound(B, kPlanQkv, kPlanHidden);
  const size_t up = gemm_partial_bound(B, kPlanQDim, kPlanRank);
  l.part_bytes = dn > up ? dn : up;
  l.chat_offset = align256(l.part_bytes);
  l.total = l.chat_offset + align256((size_t)B * kPlanRank * 2);
  return l;
}

inline size_t qproj_part_need(int B, bool bf, const GemmPlan& dn, const GemmPlan& up) {
  if (!bf) return (size_t)B * kPlanRank * sizeof(float);
  size_t n = gemm_partial_bytes(dn);
  if (up.splits > 1 && gemm_partial_bytes(up) > n) n = gemm_partial_bytes(up);
  return n;
}

// Workspace of the K/V append: fp32 partial sums of the [W_k; W_v] product.
inline size_t kv_ws_bytes(int B, bool bf) {
  return align256(bf ? gemm_partial_bound(B, 2 * kPlanHeadDim, kPlanHidden)
                     : (size_t)B * 2 * kPlanHeadDim * sizeof(float));
}
inline size_t kv_part_need(int B, bool bf, const GemmPlan& p) {
  return bf ? gemm_partial_bytes(p) : (size_t)B * 2 * kPlanHeadDim * sizeof(float);
}

// Workspace of the out-projection: fp32 partial sums when it is split.
inline size_t oproj_ws_bytes(int B, bool bf) {
  if (!bf) return 0;
  const size_t b = gemm_partial_bound(B, kPlanHidden, kPlanQDim);
  // a bound of one split means no device splits: direct output, no workspace
  return b > (size_t)B * kPlanHidden * sizeof(float) ? align256(b) : 0;
}
inline size_t oproj_part_need(bool bf, const GemmPlan& p) {
  return (bf && p.splits > 1) ? gemm_partial_bytes(p) : 0;
}

}  // namespace mfa
