// Q4_K prefill GEMM on the matrix cores: y = x * W^T, x bf16 [M][K], y fp32.
//
// Prefill over GGUF weights runs on matrix cores (hipEngine README,
// "Quickstart": WMMA prefill, GEMV decode). On gfx950 the equivalent is the
// bf16 MFMA: Q4_K tiles are decoded in fp32 (w = d*sc*q - dmin*m, exact
// products, one rounding), rounded to bf16 (nearest even) into LDS next to the
// bf16 activation tile, and contracted with v_mfma_f32_16x16x32_bf16 into fp32
// accumulators.
//
// Tiling: a 256-thread workgroup owns a BM x BN = 128 x 128 tile of y; its 4
// waves own 64 x 64 quadrants (4 x 4 MFMA tiles of 16 x 16). K advances in
// stages of 64: stage (b, c) covers code chunk c (sub-blocks 2c, 2c+1) of
// super-block b, so every stage decodes whole 32-byte code chunks. Stages are
// double-buffered in LDS; global loads for stage s+1 are issued before the
// MFMAs of stage s.
//
// MFMA operand layout (16x16x32 bf16, wave64): lane l holds, for A, row l%16
// and k = 8*(l/16) .. +7; for B, column l%16 and the same k; the 16x16 fp32
// result gives lane l column l%16 and rows 4*(l/16) .. +3.
#include "common.h"
#include "launch.h"

namespace qdm {

namespace {

constexpr int BM = 128, BN = 128, BKS = 64;
constexpr int LDS_STRIDE = BKS + 8;  // bf16 per LDS row (16-byte pad against bank conflicts)
constexpr int GEMM_THREADS = 256;

struct StageRegs {
  u32x4 xa[4];      // 4 x 16 bytes of the x tile
  u32x4 hdr, code;  // this thread's W row: block header and 16 code bytes
};

__device__ __forceinline__ void load_stage(StageRegs &r, const uint8_t *__restrict__ w,
                                           const uint16_t *__restrict__ x, int M, int N, int K,
                                           int m0, int n0, int stage) {
  const int tid = threadIdx.x;
  const int b = stage >> 2, c = stage & 3;
  const int kbase = b * QK + c * BKS;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int q = tid + GEMM_THREADS * i;
    const int row = q >> 3, col8 = (q & 7) * 8;
    const int gm = m0 + row;
    if (gm < M)
      r.xa[i] = *(const u32x4 *)(x + (int64_t)gm * K + kbase + col8);
    else
      r.xa[i] = u32x4{0, 0, 0, 0};
  }
  const int wr = tid >> 1, hf = tid & 1;
  const int gn = n0 + wr;
  if (gn < N) {
    const uint8_t *blk = w + ((int64_t)gn * (K / QK) + b) * Q4K_BYTES;
    r.hdr = *(const u32x4 *)blk;
    r.code = __builtin_nontemporal_load((const u32x4 *)(blk + 16 + 32 * c + 16 * hf));
  } else {
    r.hdr = u32x4{0, 0, 0, 0};
    r.code = u32x4{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void store_stage(const StageRegs &r, uint16_t *sx, uint16_t *sw,
                                            int stage) {
  const int tid = threadIdx.x;
  const int c = stage & 3;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int q = tid + GEMM_THREADS * i;
    const int row = q >> 3, col8 = (q & 7) * 8;
    *(u32x4 *)(sx + row * LDS_STRIDE + col8) = r.xa[i];
  }
  const int wr = tid >> 1, hf = tid & 1;
  const float d = half_bits_to_float(r.hdr.x), dmin = half_bits_to_float(r.hdr.x >> 16);
  uint32_t sc0, m0, sc1, m1;
  q4k_scale_min(r.hdr.y, r.hdr.z, r.hdr.w, 2 * c, sc0, m0);
  q4k_scale_min(r.hdr.y, r.hdr.z, r.hdr.w, 2 * c + 1, sc1, m1);
  const float a0 = d * (float)sc0, b0 = dmin * (float)m0;
  const float a1 = d * (float)sc1, b1 = dmin * (float)m1;
  const uint32_t q[4] = {r.code.x, r.code.y, r.code.z, r.code.w};
  uint32_t lo[8], hi[8];  // bf16 pairs
#pragma unroll
  for (int k = 0; k < 4; k++) {
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const uint32_t v = q[k] >> (16 * e);
      const float l0 = a0 * (float)(v & 15u) - b0;
      const float l1 = a0 * (float)((v >> 8) & 15u) - b0;
      const float h0 = a1 * (float)((v >> 4) & 15u) - b1;
      const float h1 = a1 * (float)((v >> 12) & 15u) - b1;
      lo[2 * k + e] = f32_to_bf16_rne(l0) | (f32_to_bf16_rne(l1) << 16);
      hi[2 * k + e] = f32_to_bf16_rne(h0) | (f32_to_bf16_rne(h1) << 16);
    }
  }
  uint16_t *dst = sw + wr * LDS_STRIDE + 16 * hf;
  *(u32x4 *)(dst) = u32x4{lo[0], lo[1], lo[2], lo[3]};
  *(u32x4 *)(dst + 8) = u32x4{lo[4], lo[5], lo[6], lo[7]};
  *(u32x4 *)(dst + 32) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  *(u32x4 *)(dst + 40) = u32x4{hi[4], hi[5], hi[6], hi[7]};
}

__global__ __launch_bounds__(GEMM_THREADS) void q4k_gemm_kernel(const uint8_t *__restrict__ w,
                                                                const uint16_t *__restrict__ x,
                                                                float *__restrict__ y, int M,
                                                                int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][BN * LDS_STRIDE];

  const int ntn = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / ntn) * BM, n0 = (blockIdx.x % ntn) * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int stages = (K / QK) * 4;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  StageRegs r;
  load_stage(r, w, x, M, N, K, m0, n0, 0);
  store_stage(r, sX[0], sW[0], 0);
  __syncthreads();

  const int arow = lane & 15, akoff = 8 * (lane >> 4);
  for (int s = 0; s < stages; s++) {
    const int buf = s & 1;
    if (s + 1 < stages) load_stage(r, w, x, M, N, K, m0, n0, s + 1);
    const uint16_t *sx = sX[buf], *sw = sW[buf];
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        af[i] = *(const bf16x8 *)(sx + (wm * 64 + i * 16 + arow) * LDS_STRIDE + kk * 32 + akoff);
#pragma unroll
      for (int j = 0; j < 4; j++)
        bfr[j] = *(const bf16x8 *)(sw + (wn * 64 + j * 16 + arow) * LDS_STRIDE + kk * 32 + akoff);
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < stages) store_stage(r, sX[buf ^ 1], sW[buf ^ 1], s + 1);
    __syncthreads();
  }

  const int col = lane & 15, rq = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int gn = n0 + wn * 64 + j * 16 + col;
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int gm = m0 + wm * 64 + i * 16 + rq + v;
        if (gm < M && gn < N) y[(int64_t)gm * N + gn] = acc[i][j][v];
      }
    }
}

}  // namespace

size_t q4k_gemm_workspace(int64_t, int64_t, int64_t) { return 0; }

void launch_q4k_gemm(const void *w, const void *x, float *y, int64_t M, int64_t N, int64_t K,
                     void *, hipStream_t s) {
  const dim3 grid((unsigned)(((N + BN - 1) / BN) * ((M + BM - 1) / BM)));
  hipLaunchKernelGGL(q4k_gemm_kernel, grid, dim3(GEMM_THREADS), 0, s, (const uint8_t *)w,
                     (const uint16_t *)x, y, (int)M, (int)N, (int)K);
}

}  // namespace qdm
