// Q4_K decode GEMV: y[m][n] = sum_k x[m][k] * w(n, k), M small (1..16).
//
// Decode over GGUF weights is a bandwidth-bound GEMV (hipEngine README,
// "Quickstart": GEMV decode; hipster README, hardware roofs and the GEMV
// micro-benchmark reported in GB/s). Every 144-byte super-block is read from
// HBM exactly once with 16-byte loads and decoded in registers.
//
// Work mapping (wave64):
//  * a lane owns one 32-byte code chunk c (sub-blocks 2c and 2c+1) of a
//    super-block, so 4 lanes cover a block and a wave covers 16 blocks;
//  * the 16 lane-groups of a wave are split into R = 16/G rows with G groups
//    per row, G = gcd(K/256, 16): every lane stays on one row, walks that row's
//    blocks with stride G, and no iteration is ragged;
//  * per block a lane loads the 16-byte header and its 32 code bytes.
// Arithmetic per lane and sub-block j (32 weights), with sums over the lane's
// 32 positions:
//   sum_l x_l * w_l = a_j * sum_l x_l q_l - b_j * sum_l x_l,
//   a_j = d*sc_j, b_j = dmin*m_j  (the per-sub-block scale is hoisted).
// For bf16 x the code sum uses v_dot2_f32_bf16 on exact bf16 values
// (128 + q) built with one AND-OR per two codes, then removes 128 * sum_l x_l.
// For fp32 x the codes are converted with byte-to-float conversions.
// x and its 32-element sums are staged once per workgroup in LDS; the bf16
// copy is stored with each group of four permuted to (x0, x2, x1, x3) so the
// code pairs (l, l+2), which one AND-OR extracts, meet matching x pairs.
#include "common.h"
#include "launch.h"

namespace qdm {

namespace {

constexpr int GEMV_THREADS = 256;
constexpr int GEMV_WAVES = GEMV_THREADS / WAVE;

// Stage MT rows of x into LDS. bf16: [MT][K] halves, groups of four permuted;
// fp32: [MT][K] natural. Then the 32-element sums xs[MT][K/32].
template <bool XBF16, int MT>
__device__ __forceinline__ void stage_x(const void *__restrict__ x, int K, uint32_t *lds_x,
                                        float *lds_sum) {
  const int tid = threadIdx.x;
  if constexpr (XBF16) {
    // chunks of 8 bf16 (16 bytes); 4 chunks make one 32-element sum
    const int nchunk = MT * K / 8;
    const u32x4 *src = (const u32x4 *)x;
    for (int base = 0; base < nchunk; base += GEMV_THREADS) {
      const int c = base + tid;
      float s = 0.f;
      if (c < nchunk) {
        const u32x4 v = src[c];
        // element pairs: v.x = (e0,e1), v.y = (e2,e3) -> (e0,e2), (e1,e3)
        u32x4 p;
        p.x = (v.x & 0xFFFFu) | (v.y << 16);
        p.y = (v.x >> 16) | (v.y & 0xFFFF0000u);
        p.z = (v.z & 0xFFFFu) | (v.w << 16);
        p.w = (v.z >> 16) | (v.w & 0xFFFF0000u);
        ((u32x4 *)lds_x)[c] = p;
        s = bf16_bits_to_float(v.x) + bf16_bits_to_float(v.x >> 16) +
            bf16_bits_to_float(v.y) + bf16_bits_to_float(v.y >> 16) +
            bf16_bits_to_float(v.z) + bf16_bits_to_float(v.z >> 16) +
            bf16_bits_to_float(v.w) + bf16_bits_to_float(v.w >> 16);
      }
      s += __shfl_xor(s, 1, WAVE);
      s += __shfl_xor(s, 2, WAVE);
      if (c < nchunk && (c & 3) == 0) lds_sum[c >> 2] = s;
    }
  } else {
    // chunks of 4 fp32 (16 bytes); 8 chunks make one 32-element sum
    const int nchunk = MT * K / 4;
    const f32x4 *src = (const f32x4 *)x;
    for (int base = 0; base < nchunk; base += GEMV_THREADS) {
      const int c = base + tid;
      float s = 0.f;
      if (c < nchunk) {
        const f32x4 v = src[c];
        ((f32x4 *)lds_x)[c] = v;
        s = (v.x + v.y) + (v.z + v.w);
      }
      s += __shfl_xor(s, 1, WAVE);
      s += __shfl_xor(s, 2, WAVE);
      s += __shfl_xor(s, 4, WAVE);
      if (c < nchunk && (c & 7) == 0) lds_sum[c >> 3] = s;
    }
  }
}

template <bool XBF16, int MT, int PF>
__global__ __launch_bounds__(GEMV_THREADS) void q4k_gemv_kernel(
    const uint8_t *__restrict__ w, const void *__restrict__ x, float *__restrict__ y, int N,
    int K, int G, int ldy) {
  extern __shared__ uint32_t lds[];
  uint32_t *lds_x = lds;
  float *lds_sum = (float *)(lds + (XBF16 ? MT * K / 2 : MT * K));

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 2, c = lane & 3;  // lane group (16 per wave), code chunk
  const int R = 16 / G;                   // rows per wave
  const int row = (blockIdx.x * GEMV_WAVES + wave) * R + g / G;
  const int gg = g % G;
  const int nb = K / QK;
  const int iters = nb / G;
  const bool active = row < N;
  const uint8_t *rowp = w + (int64_t)(active ? row : 0) * nb * Q4K_BYTES;

  // Per-lane constants of the scale/min decode: sub-blocks j0 = 2c, j1 = 2c+1.
  const int j0 = 2 * c;

  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; m++) acc[m] = 0.f;

  // Issue the first batch of weight loads before staging x.
  u32x4 H[PF], A[PF], B[PF];
#pragma unroll
  for (int p = 0; p < PF; p++) {
    if (active && p < iters) {
      const uint8_t *blk = rowp + (int64_t)(p * G + gg) * Q4K_BYTES;
      H[p] = __builtin_nontemporal_load((const u32x4 *)blk);
      A[p] = __builtin_nontemporal_load((const u32x4 *)(blk + 16 + 32 * c));
      B[p] = __builtin_nontemporal_load((const u32x4 *)(blk + 32 + 32 * c));
    }
  }

  stage_x<XBF16, MT>(x, K, lds_x, lds_sum);
  __syncthreads();

  if (active) {
    for (int it0 = 0; it0 < iters; it0 += PF) {
#pragma unroll
      for (int p = 0; p < PF; p++) {
        const int it = it0 + p;
        if (it < iters) {
          const int kb = it * G + gg;
          const u32x4 hdr = H[p];
          const uint32_t q[8] = {A[p].x, A[p].y, A[p].z, A[p].w,
                                 B[p].x, B[p].y, B[p].z, B[p].w};
          // prefetch the block PF iterations ahead into this slot
          if (it + PF < iters) {
            const uint8_t *blk = rowp + (int64_t)((it + PF) * G + gg) * Q4K_BYTES;
            H[p] = __builtin_nontemporal_load((const u32x4 *)blk);
            A[p] = __builtin_nontemporal_load((const u32x4 *)(blk + 16 + 32 * c));
            B[p] = __builtin_nontemporal_load((const u32x4 *)(blk + 32 + 32 * c));
          }
          const float d = half_bits_to_float(hdr.x);
          const float dmin = half_bits_to_float(hdr.x >> 16);
          uint32_t sc0, m0, sc1, m1;
          q4k_scale_min(hdr.y, hdr.z, hdr.w, j0, sc0, m0);
          q4k_scale_min(hdr.y, hdr.z, hdr.w, j0 + 1, sc1, m1);
          const float a0 = d * (float)sc0, b0 = dmin * (float)m0;
          const float a1 = d * (float)sc1, b1 = dmin * (float)m1;

          if constexpr (XBF16) {
            uint32_t np[32];
#pragma unroll
            for (int i = 0; i < 8; i++) {
              np[4 * i + 0] = nib_pair_bf16(q[i]);        // sub-block j0, l = 4i, 4i+2
              np[4 * i + 1] = nib_pair_bf16(q[i] >> 8);   // j0, 4i+1, 4i+3
              np[4 * i + 2] = nib_pair_bf16(q[i] >> 4);   // j1, 4i, 4i+2
              np[4 * i + 3] = nib_pair_bf16(q[i] >> 12);  // j1, 4i+1, 4i+3
            }
            const float c0 = fmaf(128.f, a0, b0), c1 = fmaf(128.f, a1, b1);
#pragma unroll
            for (int m = 0; m < MT; m++) {
              const u32x4 *xv = (const u32x4 *)(lds_x + (m * K + kb * QK + 32 * j0) / 2);
              const float2 xs = *(const float2 *)(lds_sum + m * (K / 32) + kb * 8 + j0);
              float s0 = 0.f, s1 = 0.f;
#pragma unroll
              for (int i = 0; i < 4; i++) {
                const u32x4 x0 = xv[i];      // j0 pairs for l = 8i .. 8i+7
                const u32x4 x1 = xv[4 + i];  // j1 pairs
                s0 = dot2_bf16(np[8 * i + 0], x0.x, s0);
                s0 = dot2_bf16(np[8 * i + 1], x0.y, s0);
                s0 = dot2_bf16(np[8 * i + 4], x0.z, s0);
                s0 = dot2_bf16(np[8 * i + 5], x0.w, s0);
                s1 = dot2_bf16(np[8 * i + 2], x1.x, s1);
                s1 = dot2_bf16(np[8 * i + 3], x1.y, s1);
                s1 = dot2_bf16(np[8 * i + 6], x1.z, s1);
                s1 = dot2_bf16(np[8 * i + 7], x1.w, s1);
              }
              float r = acc[m];
              r = fmaf(a0, s0, r);
              r = fmaf(-c0, xs.x, r);
              r = fmaf(a1, s1, r);
              r = fmaf(-c1, xs.y, r);
              acc[m] = r;
            }
          } else {
#pragma unroll
            for (int m = 0; m < MT; m++) {
              const f32x4 *xv = (const f32x4 *)((const float *)lds_x + m * K + kb * QK + 32 * j0);
              const float2 xs = *(const float2 *)(lds_sum + m * (K / 32) + kb * 8 + j0);
              float s0 = 0.f, s1 = 0.f;
#pragma unroll
              for (int i = 0; i < 8; i++) {
                const f32x4 x0 = xv[i];      // j0, l = 4i .. 4i+3
                const f32x4 x1 = xv[8 + i];  // j1
                const uint32_t lo = q[i] & 0x0F0F0F0Fu, hi = (q[i] >> 4) & 0x0F0F0F0Fu;
                s0 = fmaf(x0.x, (float)(lo & 255u), s0);
                s0 = fmaf(x0.y, (float)((lo >> 8) & 255u), s0);
                s0 = fmaf(x0.z, (float)((lo >> 16) & 255u), s0);
                s0 = fmaf(x0.w, (float)(lo >> 24), s0);
                s1 = fmaf(x1.x, (float)(hi & 255u), s1);
                s1 = fmaf(x1.y, (float)((hi >> 8) & 255u), s1);
                s1 = fmaf(x1.z, (float)((hi >> 16) & 255u), s1);
                s1 = fmaf(x1.w, (float)(hi >> 24), s1);
              }
              float r = acc[m];
              r = fmaf(a0, s0, r);
              r = fmaf(-b0, xs.x, r);
              r = fmaf(a1, s1, r);
              r = fmaf(-b1, xs.y, r);
              acc[m] = r;
            }
          }
        }
      }
    }
  }

  // Reduce over the 4G lanes of each row (aligned lane groups).
#pragma unroll
  for (int m = 0; m < MT; m++) {
    float v = group_sum(acc[m], 4 * G);
    if (active && (lane & (4 * G - 1)) == 0) y[(int64_t)m * ldy + row] = v;
  }
}

int gcd16(int nb) {
  int g = 16;
  while (g > 1 && nb % g) g >>= 1;
  return g;
}

template <bool XBF16, int MT>
void launch_chunk(const void *w, const void *x, float *y, int64_t N, int64_t K, int64_t ldy,
                  hipStream_t s) {
  const int nb = (int)(K / QK);
  const int G = gcd16(nb);
  const int R = 16 / G;
  const int64_t rows_per_wg = (int64_t)GEMV_WAVES * R;
  const unsigned grid = (unsigned)((N + rows_per_wg - 1) / rows_per_wg);
  const size_t lds = (size_t)MT * K * (XBF16 ? 2 : 4) + (size_t)MT * (K / 32) * 4;
  constexpr int PF = 2;
  auto kern = q4k_gemv_kernel<XBF16, MT, PF>;
  if (lds > 65536) hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(GEMV_THREADS), lds, s, (const uint8_t *)w, x, y,
                     (int)N, (int)K, G, (int)ldy);
}

}  // namespace

// Rows of x are processed in chunks of MT (1, 2, 4 or 8) per launch, as many
// as fit a 64 KiB LDS budget (one chunk of 1 row may use up to 136 KiB).
void launch_q4k_gemv(const void *w, const void *x, bool x_bf16, float *y, int64_t M,
                     int64_t N, int64_t K, hipStream_t s) {
  const size_t per_row = (size_t)K * (x_bf16 ? 2 : 4) + (size_t)(K / 32) * 4;
  const size_t elt = x_bf16 ? 2 : 4;
  int64_t m0 = 0;
  while (m0 < M) {
    const int64_t rem = M - m0;
    int mt = 8;
    while (mt > 1 && (mt > rem || (size_t)mt * per_row > 65536)) mt >>= 1;
    const void *xm = (const char *)x + (size_t)m0 * K * elt;
    float *ym = y + m0 * N;
    if (x_bf16) {
      switch (mt) {
        case 8: launch_chunk<true, 8>(w, xm, ym, N, K, N, s); break;
        case 4: launch_chunk<true, 4>(w, xm, ym, N, K, N, s); break;
        case 2: launch_chunk<true, 2>(w, xm, ym, N, K, N, s); break;
        default: launch_chunk<true, 1>(w, xm, ym, N, K, N, s); break;
      }
    } else {
      switch (mt) {
        case 8: launch_chunk<false, 8>(w, xm, ym, N, K, N, s); break;
        case 4: launch_chunk<false, 4>(w, xm, ym, N, K, N, s); break;
        case 2: launch_chunk<false, 2>(w, xm, ym, N, K, N, s); break;
        default: launch_chunk<false, 1>(w, xm, ym, N, K, N, s); break;
      }
    }
    m0 += mt;
  }
}

}  // namespace qdm
