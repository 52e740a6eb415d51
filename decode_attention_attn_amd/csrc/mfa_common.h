// Shared device-side definitions for the libmfa kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfa {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define MFA_LDS __attribute__((address_space(3)))

constexpr int kHidden = 7168;
constexpr int kRank = 2048;
constexpr int kHeads = 64;
constexpr int kHeadDim = 256;
constexpr int kQDim = kHeads * kHeadDim;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 4 e4m3fn bytes of a dword -> 4 bf16 (exact: every e4m3 value is a bf16 value).
__device__ __forceinline__ void fp8x4_to_bf16(unsigned w, bf16x8& dst, int at) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  dst[at + 0] = lo[0];
  dst[at + 1] = lo[1];
  dst[at + 2] = hi[0];
  dst[at + 3] = hi[1];
}

// Values every lane of the wave already agrees on, made provably uniform so
// the compiler keeps them (and loads indexed by them) in scalar registers.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ long long uniform(long long x) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)x);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Load through the constant address space: with a uniform index this becomes a
// scalar (s_load) read, which is tracked by lgkmcnt and so never waits on the
// vector-memory counter that the LDS DMA ring relies on. Only for data the
// kernel does not write.
template <typename T>
__device__ __forceinline__ T load_scalar(const T* p, long long i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// gfx950 transposing LDS reads. The __restrict__ parameter gives the inlined
// read alias-scope metadata; without it the compiler cannot tell the read from
// the in-flight direct-to-LDS loads and waits for all of them (vmcnt(0)) before
// every read, which would serialize the DMA ring. Completion of the tile being
// read is ensured explicitly (vmcnt wait + barrier) by the callers.
__device__ __forceinline__ bf16x4 lds_read_tr16(const MFA_LDS bf16x4* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MFA_LDS bf16x4*)p);
}
__device__ __forceinline__ i32x2 lds_read_tr8(const MFA_LDS i32x2* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((MFA_LDS i32x2*)p);
}
// Plain 16-byte LDS read with the same alias-scope treatment.
__device__ __forceinline__ bf16x8 lds_read_b128(const MFA_LDS bf16x8* __restrict__ p) { return *p; }

// Cross-lane combine of the 4 lanes n, n+16, n+32, n+48 (one value per
// 16-lane row) with the gfx950 row/half swaps: no LDS round trip.
__device__ __forceinline__ float max_over_rows(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(r[0]) + __int_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Wave-wide reductions over all 64 lanes.
__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace mfa
