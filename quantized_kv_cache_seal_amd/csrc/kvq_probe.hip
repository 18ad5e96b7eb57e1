// Streaming read of a device buffer, for measurement only: the achievable
// HBM read rate of this device, next to which the decode's roofline fraction
// (against the 8 TB/s peak) can be read.  Not part of the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_layout.h"

namespace kvq {

// Grid-stride 16-byte non-temporal loads, eight in flight per thread, folded by
// XOR into one word per wave (written to out[4 blockIdx.x + wave]) so that
// none of them can be dropped.  The fastest of the forms measured (1,024 to
// 16,384 workgroups, 4 to 16 loads in flight, ordinary or non-temporal loads):
// 6.8 TB/s over 4 GiB.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4v* __restrict__ src, int64_t n16, uint32_t* out) {
  constexpr int U = 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4v v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4v v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) out[4 * blockIdx.x + (threadIdx.x >> 6)] = acc;
}

hipError_t launch_read_probe(const void* src, int64_t bytes, void* out, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kReadProbeBlocks), dim3(256), 0, stream, (const u32x4v*)src, bytes / 16,
                     (uint32_t*)out);
  return hipGetLastError();
}

}  // namespace kvq
