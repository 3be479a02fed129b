// Pieces shared by the Q4_K / Q5_K matrix-core kernels (gfx950): the LDS row
// pitch of the GEMM's x tile, bf16 packing, and a block header's sub-block
// scales. Both kernels decode w = d*sc*q - dmin*m in fp32 (the product is
// exact, so there is one rounding) and round it to bf16 nearest-even
// (v_cvt_pk_bf16_f32) in registers, straight into the MFMA operand.
#pragma once

#include "common.h"

namespace qdm {
namespace {

constexpr int TILE_LROW = 64 + 8;  // bf16 per LDS row: 64 values + 16 bytes of bank padding

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Scales of a code chunk's two sub-blocks for one weight row.
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

}  // namespace
}  // namespace qdm
