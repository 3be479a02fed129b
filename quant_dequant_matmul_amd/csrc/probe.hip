// Streaming copy of a known number of bytes: the calibration kernel for
// memory-traffic counters and the achievable-HBM-bandwidth probe (the hipster
// README reports such measured roofs for its own device).
#include "common.h"
#include "launch.h"

namespace qdm {

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4 *__restrict__ src,
                                                         u32x4 *__restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

void launch_probe_copy(const void *src, void *dst, int64_t n_bytes, hipStream_t s) {
  const int64_t n16 = n_bytes / 16;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const u32x4 *)src, (u32x4 *)dst, n16);
}

}  // namespace qdm
