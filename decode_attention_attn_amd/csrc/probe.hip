// Streaming-read bandwidth probe: the achievable HBM read rate that the
// attention kernels' KV rate is compared with. Every workgroup reads a
// grid-strided share of the buffer with nontemporal 16-byte vector loads
// (eight in flight per thread), XORs what it read and writes one 32-bit
// checksum, so the loads cannot be dropped and the result can be checked
// exactly. One workgroup per CU measured fastest on MI355X (7.1 TB/s over
// 4 GiB, against 5.8 with four per CU and 6.3 with plain loads).

#include "mfa_common.h"
#include "mfa_internal.h"

namespace mfa {

__global__ __launch_bounds__(256) void bw_probe_kernel(const u32x4* __restrict__ buf, long long n16,
                                                       unsigned* __restrict__ sink) {
  const long long stride = (long long)gridDim.x * 256;
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(buf + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
  unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x ^= __shfl_xor(x, d);
  __shared__ unsigned part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

hipError_t launch_bw_probe(const void* buf, size_t bytes, unsigned* sink, int G, hipStream_t stream) {
  return launch(bw_probe_kernel, dim3(G), dim3(256), stream, (const u32x4*)buf, (long long)(bytes / 16), sink);
}

}  // namespace mfa
