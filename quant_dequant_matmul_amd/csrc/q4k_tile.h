// Q4_K (and Q5_K) tile decode shared by the matrix-core kernels (gfx950): one thread
// owns one weight row of a 256-row tile and, per K stage of 64, decodes code
// chunk c of a super-block (sub-blocks 2c and 2c+1) into bf16 LDS slots in
// MFMA operand order. w = d*sc*q - dmin*m is formed in fp32 (the product is
// exact, so there is one rounding) and rounded to bf16 nearest-even
// (v_cvt_pk_bf16_f32).
#pragma once

#include "common.h"

namespace qdm {
namespace {

constexpr int TILE_LROW = 64 + 8;  // bf16 per LDS row: 64 weights + 16 bytes of bank padding

struct WRegs {
  u32x4 hdr, qa, qb;  // this thread's W row: block header and 32 code bytes
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Scales of the stage's two sub-blocks for this thread's W row.
struct RowScales {
  float a0, b0, a1, b1;
};

// From a block's 16-byte header (d, dmin, packed scales): the scales of code
// chunk c's two sub-blocks; all zero for a row past N.
__device__ __forceinline__ RowScales hdr_scales(const u32x4 &hdr, bool live, int c) {
  const float d = live ? half_bits_to_float(hdr.x) : 0.f;
  const float dmin = live ? half_bits_to_float(hdr.x >> 16) : 0.f;
  uint32_t sc0, m0s, sc1, m1s;
  q4k_scale_min(hdr.y, hdr.z, hdr.w, 2 * c, sc0, m0s);
  q4k_scale_min(hdr.y, hdr.z, hdr.w, 2 * c + 1, sc1, m1s);
  return RowScales{d * (float)sc0, dmin * (float)m0s, d * (float)sc1, dmin * (float)m1s};
}

__device__ __forceinline__ RowScales row_scales(const WRegs &r, bool live, int c) {
  return hdr_scales(r.hdr, live, c);
}

// Part kk (0..3) of a W row's decode: code dwords 2kk, 2kk+1, i.e. positions
// 8kk .. 8kk+7 of both sub-blocks, stored as bf16 into the row's LDS slots.
__device__ __forceinline__ void store_w_part(const WRegs &r, const RowScales &sc, int kk,
                                             uint16_t *sw) {
  const uint32_t qd[2] = {kk < 2 ? r.qa[2 * kk] : r.qb[2 * kk - 4],
                          kk < 2 ? r.qa[2 * kk + 1] : r.qb[2 * kk - 3]};
  uint32_t lo[4], hi[4];
  // an opaque mask keeps the nibbles byte-aligned, so each code converts with
  // one v_cvt_f32_ubyteN instead of a field extract plus a conversion
  uint32_t nib = 0x0F0F0F0Fu;
  asm volatile("" : "+v"(nib));
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const uint32_t l4 = qd[u] & nib, h4 = (qd[u] >> 4) & nib;
    lo[2 * u] = pack_bf16(sc.a0 * (float)(l4 & 255u) - sc.b0,
                          sc.a0 * (float)((l4 >> 8) & 255u) - sc.b0);
    lo[2 * u + 1] = pack_bf16(sc.a0 * (float)((l4 >> 16) & 255u) - sc.b0,
                              sc.a0 * (float)(l4 >> 24) - sc.b0);
    hi[2 * u] = pack_bf16(sc.a1 * (float)(h4 & 255u) - sc.b1,
                          sc.a1 * (float)((h4 >> 8) & 255u) - sc.b1);
    hi[2 * u + 1] = pack_bf16(sc.a1 * (float)((h4 >> 16) & 255u) - sc.b1,
                              sc.a1 * (float)(h4 >> 24) - sc.b1);
  }
  uint16_t *dst = sw + threadIdx.x * TILE_LROW;
  *(u32x4 *)(dst + 8 * kk) = u32x4{lo[0], lo[1], lo[2], lo[3]};
  *(u32x4 *)(dst + 32 + 8 * kk) = u32x4{hi[0], hi[1], hi[2], hi[3]};
}

// Q5_K variant of store_w_part: the code words come from the block's code
// bytes at 48 (wr.qa, wr.qb hold chunk c as for Q4_K) and the fifth bits from
// the 32-byte high-bit plane (qh0 = bytes 0..15, qh1 = 16..31): bit 2c of byte
// l for the low-nibble sub-block, bit 2c+1 for the high-nibble one.
__device__ __forceinline__ void store_w_part5(const WRegs &r, const u32x4 &qh0, const u32x4 &qh1,
                                              const RowScales &sc, int kk, int c, uint16_t *sw) {
  const uint32_t qd[2] = {kk < 2 ? r.qa[2 * kk] : r.qb[2 * kk - 4],
                          kk < 2 ? r.qa[2 * kk + 1] : r.qb[2 * kk - 3]};
  const uint32_t hq[2] = {kk < 2 ? qh0[2 * kk] : qh1[2 * kk - 4],
                          kk < 2 ? qh0[2 * kk + 1] : qh1[2 * kk - 3]};
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const uint32_t hh = hq[u] >> (2 * c);
    const uint32_t l5 = (qd[u] & 0x0F0F0F0Fu) | ((hh << 4) & 0x10101010u);
    const uint32_t h5 = ((qd[u] >> 4) & 0x0F0F0F0Fu) | ((hh << 3) & 0x10101010u);
    lo[2 * u] = pack_bf16(sc.a0 * (float)(l5 & 255u) - sc.b0,
                          sc.a0 * (float)((l5 >> 8) & 255u) - sc.b0);
    lo[2 * u + 1] = pack_bf16(sc.a0 * (float)((l5 >> 16) & 255u) - sc.b0,
                              sc.a0 * (float)(l5 >> 24) - sc.b0);
    hi[2 * u] = pack_bf16(sc.a1 * (float)(h5 & 255u) - sc.b1,
                          sc.a1 * (float)((h5 >> 8) & 255u) - sc.b1);
    hi[2 * u + 1] = pack_bf16(sc.a1 * (float)((h5 >> 16) & 255u) - sc.b1,
                              sc.a1 * (float)(h5 >> 24) - sc.b1);
  }
  uint16_t *dst = sw + threadIdx.x * TILE_LROW;
  *(u32x4 *)(dst + 8 * kk) = u32x4{lo[0], lo[1], lo[2], lo[3]};
  *(u32x4 *)(dst + 32 + 8 * kk) = u32x4{hi[0], hi[1], hi[2], hi[3]};
}

}  // namespace
}  // namespace qdm
