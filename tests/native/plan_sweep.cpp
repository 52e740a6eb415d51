// Host-only check of the projection workspace sizing: for every batch size
// in a sweep and every compute-unit count 1..256, the plan a device would
// make must fit the region a workspace query reserves without a device.
// Prints one line per violation and exits non-zero if there is any.
#include <stdio.h>

#include "plan.h"

int main() {
  using namespace mfa;
  long bad = 0, checked = 0;
  int batches[600];
  int nb = 0;
  for (int b = 1; b <= 300; ++b) batches[nb++] = b;
  for (int b = 301; b <= 65536 && nb < 600; b = b * 5 / 4 + 1) batches[nb++] = b;
  for (int i = 0; i < nb; ++i) {
    const int B = batches[i];
    for (int bf = 0; bf < 2; ++bf) {
      const QprojLayout ql = qproj_layout(B, bf);
      const size_t kv = kv_ws_bytes(B, bf);
      const size_t op = oproj_ws_bytes(B, bf);
      if (ql.chat_offset < ql.part_bytes || ql.total < ql.chat_offset + (size_t)B * kPlanRank * (bf ? 2 : 4)) {
        printf("q layout overlaps: B=%d bf=%d\n", B, bf);
        ++bad;
      }
      // bf16 weights and (bf16 activations only) block-fp8 weights
      for (int w8 = 0; w8 <= bf; ++w8)
        for (int cus = 1; cus <= kPlanCus; ++cus) {
          const GemmPlan dn = plan_gemm(bf, B, kPlanRank, kPlanHidden, kPlanRank, cus, w8);
          const GemmPlan up = plan_gemm(bf, B, kPlanQDim, kPlanRank, kPlanQDim, cus, w8);
          const GemmPlan kp = plan_gemm(bf, B, 2 * kPlanHeadDim, kPlanHidden, kPlanHeadDim, cus, w8);
          const GemmPlan opl = plan_gemm(bf, B, kPlanHidden, kPlanQDim, kPlanHidden, cus, w8);
          const size_t q_need = qproj_part_need(B, bf, dn, up);
          if (q_need > ql.part_bytes) {
            printf("q path: B=%d bf=%d w8=%d cus=%d needs %zu > %zu\n", B, bf, w8, cus, q_need, ql.part_bytes);
            ++bad;
          }
          if (kv_part_need(B, bf, kp) > kv) {
            printf("kv: B=%d bf=%d w8=%d cus=%d needs %zu > %zu\n", B, bf, w8, cus, kv_part_need(B, bf, kp), kv);
            ++bad;
          }
          if (oproj_part_need(bf, opl) > op) {
            printf("oproj: B=%d bf=%d w8=%d cus=%d needs %zu > %zu\n", B, bf, w8, cus, oproj_part_need(bf, opl), op);
            ++bad;
          }
          // a plan's tile divides its columns (the launcher rejects it otherwise)
          const GemmPlan all[4] = {dn, up, kp, opl};
          for (const GemmPlan& g : all)
            if (bf && (g.N % g.tile_n != 0 || (w8 ? (g.tile_n != 128 && g.tile_n != 256)
                                                   : (g.tile_n != 64 && g.tile_n != 128)))) {
              printf("tile: B=%d w8=%d cus=%d N=%d tile %d\n", B, w8, cus, g.N, g.tile_n);
              ++bad;
            }
          checked += 3;
        }
    }
    // the q path with the K/V projections folded in (bf16 activations, either weight format)
    const QprojLayout qk = qkv_layout(B);
    if (qk.chat_offset < qk.part_bytes || qk.total < qk.chat_offset + (size_t)B * kPlanRank * 2) {
      printf("qkv layout overlaps: B=%d\n", B);
      ++bad;
    }
    for (int w8 = 0; w8 < 2; ++w8)
      for (int cus = 1; cus <= kPlanCus; ++cus) {
        const GemmPlan dn = plan_gemm(true, B, kPlanQkv, kPlanHidden, kPlanRank, cus, w8);
        const GemmPlan up = plan_gemm(true, B, kPlanQDim, kPlanRank, kPlanQDim, cus, w8);
        const size_t need = qproj_part_need(B, true, dn, up);
        if (need > qk.part_bytes) {
          printf("qkv: B=%d w8=%d cus=%d needs %zu > %zu\n", B, w8, cus, need, qk.part_bytes);
          ++bad;
        }
        if (dn.N % dn.tile_n != 0 || up.N % up.tile_n != 0) {
          printf("qkv tile: B=%d w8=%d cus=%d tiles %d / %d\n", B, w8, cus, dn.tile_n, up.tile_n);
          ++bad;
        }
        ++checked;
      }
  }
  printf("checked %ld plans, %ld over their workspace\n", checked, bad);
  return bad == 0 ? 0 : 1;
}
