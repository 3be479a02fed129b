// Bit-exact dequantization of packed Q4_K / Q5_K / Q6_K tensors to fp32 [N][K].
//
// Weight formulas (GGUF k-quant tensor families named in the hipEngine README,
// "GGUF Support"): Q4_K and Q5_K w = d*sc_j*q - dmin*m_j (Q5_K codes carry a
// fifth bit from a 32-byte high-bit plane); Q6_K w = d*scale*(q-32).
// Every product is exact in fp32, so computing them in fp32 and subtracting
// once gives the correctly rounded value whatever the evaluation order.
#include "common.h"
#include "launch.h"

namespace qdm {

// One thread per 8 consecutive weights of one super-block (32 threads/block).
__global__ __launch_bounds__(256) void q4k_dequant_kernel(const uint8_t *__restrict__ w,
                                                          float *__restrict__ out,
                                                          int64_t nblocks) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = t >> 5;
  if (blk >= nblocks) return;
  const int i = (int)(t & 31);
  const uint8_t *B = w + blk * Q4K_BYTES;
  const u32x4 hdr = *(const u32x4 *)B;
  const float d = half_bits_to_float(hdr.x), dmin = half_bits_to_float(hdr.x >> 16);
  const int j = i >> 2, l0 = (i & 3) * 8;
  uint32_t sc, m;
  q4k_scale_min(hdr.y, hdr.z, hdr.w, j, sc, m);
  const float a = d * (float)sc, b = dmin * (float)m;
  const u32x2 q = *(const u32x2 *)(B + 16 + 32 * (j >> 1) + l0);
  const int sh = 4 * (j & 1);
  f32x4 r0, r1;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    r0[e] = a * (float)((q.x >> (8 * e + sh)) & 15u) - b;
    r1[e] = a * (float)((q.y >> (8 * e + sh)) & 15u) - b;
  }
  // out is [N][K] with K = 256 * (blocks per row): block blk starts at blk*256.
  f32x4 *o = (f32x4 *)(out + blk * QK + 32 * j + l0);
  o[0] = r0;
  o[1] = r1;
}

// Q5_K: as Q4_K, with the codes at byte 48 and the fifth bit of weight l of
// sub-block j in bit j of high-bit byte 16 + l.
__global__ __launch_bounds__(256) void q5k_dequant_kernel(const uint8_t *__restrict__ w,
                                                          float *__restrict__ out,
                                                          int64_t nblocks) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = t >> 5;
  if (blk >= nblocks) return;
  const int i = (int)(t & 31);
  const uint8_t *B = w + blk * Q5K_BYTES;
  const u32x4 hdr = *(const u32x4 *)B;
  const float d = half_bits_to_float(hdr.x), dmin = half_bits_to_float(hdr.x >> 16);
  const int j = i >> 2, l0 = (i & 3) * 8;
  uint32_t sc, m;
  q4k_scale_min(hdr.y, hdr.z, hdr.w, j, sc, m);
  const float a = d * (float)sc, b = dmin * (float)m;
  const u32x2 q = *(const u32x2 *)(B + 48 + 32 * (j >> 1) + l0);
  const u32x2 qh = *(const u32x2 *)(B + 16 + l0);
  const int sh = 4 * (j & 1);
  f32x4 r0, r1;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const uint32_t q0 = ((q.x >> (8 * e + sh)) & 15u) | (((qh.x >> (8 * e + j)) & 1u) << 4);
    const uint32_t q1 = ((q.y >> (8 * e + sh)) & 15u) | (((qh.y >> (8 * e + j)) & 1u) << 4);
    r0[e] = a * (float)q0 - b;
    r1[e] = a * (float)q1 - b;
  }
  f32x4 *o = (f32x4 *)(out + blk * QK + 32 * j + l0);
  o[0] = r0;
  o[1] = r1;
}

// One thread per 8 consecutive weights. Weight i of a block: h = i/128,
// g = (i%128)/32, l = i%32; low nibble from QL[64h + 32(g%2) + l] (high half
// when g >= 2), high pair from bits 2g..2g+1 of QH[32h + l], scale i/16.
// Blocks are 210 bytes, so only 2-byte alignment holds: bytes are read singly.
__global__ __launch_bounds__(256) void q6k_dequant_kernel(const uint8_t *__restrict__ w,
                                                          float *__restrict__ out,
                                                          int64_t nblocks) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = t >> 5;
  if (blk >= nblocks) return;
  const int i0 = (int)(t & 31) * 8;
  const uint8_t *B = w + blk * Q6K_BYTES;
  const int h = i0 >> 7, r = i0 & 127, g = r >> 5, l0 = r & 31;
  const uint8_t *ql = B + 64 * h + 32 * (g & 1) + l0;
  const uint8_t *qh = B + 128 + 32 * h + l0;
  const float d = half_bits_to_float((uint32_t)B[208] | ((uint32_t)B[209] << 8));
  const float a = d * (float)(int8_t)B[192 + (i0 >> 4)];
  const int shl = 4 * (g >> 1), shh = 2 * g;
  f32x4 r0, r1;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const int q = ((ql[e] >> shl) & 15) | (((qh[e] >> shh) & 3) << 4);
    const float v = a * (float)(q - 32);
    if (e < 4) r0[e] = v; else r1[e - 4] = v;
  }
  f32x4 *o = (f32x4 *)(out + blk * QK + i0);
  o[0] = r0;
  o[1] = r1;
}

void launch_q4k_dequantize(const void *w, float *out, int64_t N, int64_t K, hipStream_t s) {
  const int64_t nblocks = N * (K / QK);
  const int64_t threads = nblocks * 32;
  hipLaunchKernelGGL(q4k_dequant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, (const uint8_t *)w, out, nblocks);
}

void launch_q5k_dequantize(const void *w, float *out, int64_t N, int64_t K, hipStream_t s) {
  const int64_t nblocks = N * (K / QK);
  const int64_t threads = nblocks * 32;
  hipLaunchKernelGGL(q5k_dequant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, (const uint8_t *)w, out, nblocks);
}

void launch_q6k_dequantize(const void *w, float *out, int64_t N, int64_t K, hipStream_t s) {
  const int64_t nblocks = N * (K / QK);
  const int64_t threads = nblocks * 32;
  hipLaunchKernelGGL(q6k_dequant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, (const uint8_t *)w, out, nblocks);
}

}  // namespace qdm
