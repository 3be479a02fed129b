// Device-side helpers shared by the kernels of libqdm (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qdm {

constexpr int QK = 256;          // weights per super-block
constexpr int Q4K_BYTES = 144;   // Q4_K super-block
constexpr int Q5K_BYTES = 176;   // Q5_K super-block: Q4_K header, 32 high-bit bytes, 128 code bytes
constexpr int Q6K_BYTES = 210;   // Q6_K super-block
constexpr int Q80_BYTES = 34;    // Q8_0 block: fp16 d, 32 int8 codes
constexpr int WAVE = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp16 bit pattern (low 16 bits of h) -> fp32, exact (v_cvt_f32_f16).
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}

// bf16 bit pattern -> fp32, exact.
__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __builtin_bit_cast(float, (b & 0xFFFFu) << 16);
}

// Unsigned bitfield extract (v_bfe_u32): (v >> off) & ((1 << width) - 1),
// width 0 gives 0.
__device__ __forceinline__ uint32_t bfe(uint32_t v, uint32_t off, uint32_t width) {
  return __builtin_amdgcn_ubfe(v, off, width);
}

// Two bf16 products accumulated into an fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Two 4-bit codes at bits 0..3 and 16..19 of u, as the bf16 pair
// (128 + q_lo, 128 + q_hi): 0x43 in the high byte of a bf16 is the exponent of
// 128 with a mantissa step of exactly 1, so the nibble lands as an exact
// integer offset from 128.
__device__ __forceinline__ uint32_t nib_pair_bf16(uint32_t u) {
  return (u & 0x000F000Fu) | 0x43004300u;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Sum over aligned groups of N = 2, 4 or 8 lanes, in every lane, with DPP
// lane swaps (no LDS permute): neighbours, then pairs within a quad, then the
// mirrored half row (lane i with 7 - i, which holds the other quad's sum).
// Each step adds a lane's value and its partner's, as the xor butterfly
// does, so the bits equal those of s += __shfl_xor(s, 1), (s, 2), (s, 4).
// Every lane of the wave must be active.
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(N == 2 || N == 4 || N == 8, "groups of 2, 4 or 8 lanes");
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  if constexpr (N >= 4)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  if constexpr (N >= 8)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

// Sum over the 64 lanes of a wave (result valid in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Q4_K sub-block scale and min of sub-block j from the 12 packed bytes given
// as three little-endian words S0 = bytes 0..3, S1 = 4..7, S2 = 8..11.
//   j < 4 : sc = S[j] & 63,                    m = S[j+4] & 63
//   j >= 4: sc = (S[j+4] & 15) | (S[j-4] >> 6) << 4,
//           m  = (S[j+4] >> 4) | (S[j]   >> 6) << 4
__device__ __forceinline__ void q4k_scale_min(uint32_t S0, uint32_t S1, uint32_t S2,
                                              int j, uint32_t &sc, uint32_t &m) {
  if (j < 4) {
    sc = bfe(S0, 8 * j, 6);
    m = bfe(S1, 8 * j, 6);
  } else {
    const int jj = j - 4;
    sc = bfe(S2, 8 * jj, 4) | (bfe(S0, 8 * jj + 6, 2) << 4);
    m = bfe(S2, 8 * jj + 4, 4) | (bfe(S1, 8 * jj + 6, 2) << 4);
  }
}

}  // namespace qdm
