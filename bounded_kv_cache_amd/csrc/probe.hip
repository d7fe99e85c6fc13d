// HBM read-bandwidth probe: a plain streaming read of one buffer, the measured
// ceiling the decode kernel is compared against next to the published peak.
// One workgroup per CU streams a contiguous share of the buffer with sixteen
// 16-byte non-temporal loads in flight per thread (of the layouts tried --
// grid-stride or contiguous shares, 1 to 8 workgroups per CU, 4 to 32 loads
// in flight -- this one read fastest), and every word is folded into one XOR
// checksum so no load can be dropped.
#include "ps_internal.h"

namespace ps {
namespace {

constexpr int kProbeInFlight = 16;

__global__ __launch_bounds__(64) void probe_zero_kernel(uint32_t* out) {
  if (threadIdx.x == 0) *out = 0u;
}

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* src, int64_t n16, uint32_t* out) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
  int64_t i = b0 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kProbeInFlight - 1) * 256 < b1; i += kProbeInFlight * 256) {
    u32x4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) acc ^= v[u];
  }
  for (; i < b1; i += 256) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = 32; off > 0; off >>= 1) v ^= __shfl_xor(v, off);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) atomicXor(out, part[0] ^ part[1] ^ part[2] ^ part[3]);
}

}  // namespace

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* checksum, int cu_count, hipStream_t stream) {
  hipLaunchKernelGGL(probe_zero_kernel, dim3(1), dim3(64), 0, stream, checksum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || bytes == 0) return e;
  const int64_t n16 = bytes / 16;
  int64_t blocks = (n16 + 255) / 256;
  const int64_t cap = cu_count > 0 ? cu_count : 256;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(read_probe_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), n16, checksum);
  return hipGetLastError();
}

}  // namespace ps
