// Roofline probes: plain kernels of known work that measure what this device
// actually sustains, reported beside the nominal peaks (the hipster README,
// "Hardware and software this was measured on", lists such measured roofs:
// DRAM read, per-launch cost and bf16 GEMM).
//  * probe_copy: streaming copy of a known byte count, also the calibration
//    kernel of the memory-traffic counters;
//  * probe_read: read-only stream (every byte read once, a contiguous slice
//    per workgroup, 16-byte non-temporal loads, four 4 KiB steps in flight);
//  * probe_mfma: back-to-back bf16 MFMAs (v_mfma_f32_32x32x16_bf16, eight
//    independent accumulators per wave) with the shader clock and the
//    100 MHz reference clock read around the loop;
//  * probe_empty: a launch that does nothing (per-launch cost).
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

// Workgroup b reads its own contiguous slice of the buffer front to back, a
// 4 KiB step per iteration (256 threads x 16 bytes, non-temporal), four steps
// in flight. Reading a contiguous slice per workgroup sustains about 7 TB/s
// on MI355X; a grid-stride walk (every thread's loads spread over the whole
// buffer) topped out near 5.6 TB/s at 2048 workgroups. The xor of everything
// read decides a store that practically never happens (sink must be a valid
// 4-byte buffer all the same), so no load is dropped.
constexpr int PR_THREADS = 256, PR_STEPS = 4, PR_WGS = 1024;
__global__ __launch_bounds__(PR_THREADS) void probe_read_kernel(const u32x4 *__restrict__ src,
                                                                int64_t n16, uint32_t *__restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = b0 + threadIdx.x;
  for (; i + (PR_STEPS - 1) * PR_THREADS < b1; i += PR_STEPS * PR_THREADS) {
    u32x4 v[PR_STEPS];
#pragma unroll
    for (int u = 0; u < PR_STEPS; u++) v[u] = __builtin_nontemporal_load(src + i + u * PR_THREADS);
#pragma unroll
    for (int u = 0; u < PR_STEPS; u++) acc ^= v[u];
  }
  for (; i < b1; i += PR_THREADS) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t v = (acc.x ^ acc.y) ^ (acc.z ^ acc.w);
  if (v == 0x9E3779B9u) sink[0] = v;
}

void launch_probe_read(const void *src, int64_t n_bytes, uint32_t *sink, hipStream_t s) {
  const int64_t n16 = n_bytes / 16;
  int64_t blocks = (n16 + PR_THREADS - 1) / PR_THREADS;  // at least one 4 KiB step each
  if (blocks > PR_WGS) blocks = PR_WGS;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(PR_THREADS), 0, s,
                     (const u32x4 *)src, n16, sink);
}

// Each wave: iters x 8 MFMAs of 32 x 32 x 16 (32768 flops each). Operands
// come from the lane index so nothing folds; the sum of the accumulators
// decides a store that never happens (the values stay small and finite).
// Wave 0 of every workgroup writes its shader-clock and reference-clock
// deltas to clocks[2 * workgroup] and [2 * workgroup + 1].
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float *__restrict__ sink,
                                                         uint64_t *__restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    a[j] = (__bf16)(0.0078125f * (float)((lane + j) & 7));
    b[j] = (__bf16)(0.0078125f * (float)((lane * 3 + j) & 7));
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; j++)
#pragma unroll
    for (int v = 0; v < 16; v++) acc[j][v] = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < 8; j++) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j++)
#pragma unroll
    for (int v = 0; v < 16; v++) sum += acc[j][v];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (sum == -1.f) sink[0] = sum;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

void launch_probe_mfma(int64_t iters, int64_t workgroups, float *sink, uint64_t *clocks,
                       hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, (int)iters,
                     sink, clocks);
}

__global__ __launch_bounds__(64) void probe_empty_kernel() {}

void launch_probe_empty(int64_t workgroups, hipStream_t s) {
  hipLaunchKernelGGL(probe_empty_kernel, dim3((unsigned)workgroups), dim3(64), 0, s);
}

}  // namespace qdm
