// Q4_K decode GEMV: y[m][n] = sum_k x[m][k] * w(n, k), M small (1..16).
//
// Decode over GGUF weights is a bandwidth-bound GEMV (hipEngine README,
// "Quickstart": GEMV decode; hipster README, hardware roofs and the GEMV
// micro-benchmark reported in GB/s). Every 144-byte super-block is read from
// HBM exactly once with 16-byte loads and decoded in registers.
//
// Work split (balanced for any K):
//  * workgroup b owns rows [r0, r1) (row counts differ by at most one), i.e.
//    the contiguous block range [r0*nb, r1*nb) of the tensor (nb = K/256);
//  * its waves split that block range evenly; one wave iteration covers 16
//    consecutive blocks, 4 lanes per block, and a lane owns one 32-byte code
//    chunk c (sub-blocks 2c and 2c+1) of its block;
//  * each block's contribution (summed over its 4 lanes) goes to an LDS slot,
//    and the workgroup finally sums each row's slots in block order, so the
//    result does not depend on timing (bitwise deterministic).
// Arithmetic per lane and sub-block j (32 weights, sums over its positions):
//   sum_l x_l * w_l = a_j * sum_l x_l q_l - b_j * sum_l x_l,
//   a_j = d*sc_j, b_j = dmin*m_j  (per-sub-block scale hoisted out).
// bf16 x: two codes become the exact bf16 values (128 + q_l, 128 + q_l+2) with
// one v_and_or_b32 (0x43 in a bf16's high byte is the exponent of 128 with a
// mantissa step of 1), multiplied with v_dot2_f32_bf16 against x pairs
// (x_l, x_l+2), and 128 * sum_l x_l is removed with the sub-block x sum.
// fp32 x: codes are converted with byte-to-float conversions.
// x and its 32-element sums are staged in LDS once per workgroup; the bf16
// copy stores each group of four as (x0, x2, x1, x3) to match the code pairs.
#include "common.h"
#include "launch.h"

namespace qdm {

namespace {

constexpr int GV_THREADS = 256;
constexpr int GV_WAVES = GV_THREADS / WAVE;
constexpr int GV_PF = 4;  // wave iterations of loads kept in flight
constexpr int GV_TARGET_WGS = 1024;  // 4 per compute unit

// A value the compiler cannot see through, so it stays in a VGPR and the
// AND-OR below is formed as one v_and_or_b32 (VOP3 takes no literals here).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <bool XBF16, int MT>
__device__ __forceinline__ void stage_x(const void *__restrict__ x, int K, uint32_t *lds_x,
                                        float *lds_sum) {
  const int tid = threadIdx.x;
  if constexpr (XBF16) {
    const int nchunk = MT * K / 8;  // 8 bf16 per chunk, 4 chunks per 32-sum
    const u32x4 *src = (const u32x4 *)x;
    for (int base = 0; base < nchunk; base += GV_THREADS) {
      const int c = base + tid;
      float s = 0.f;
      if (c < nchunk) {
        const u32x4 v = src[c];
        u32x4 p;  // (e0,e1),(e2,e3) -> (e0,e2),(e1,e3)
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
      s = lane_group_sum<4>(s);
      if (c < nchunk && (c & 3) == 0) lds_sum[c >> 2] = s;
    }
  } else {
    const int nchunk = MT * K / 4;  // 4 fp32 per chunk, 8 chunks per 32-sum
    const f32x4 *src = (const f32x4 *)x;
    for (int base = 0; base < nchunk; base += GV_THREADS) {
      const int c = base + tid;
      float s = 0.f;
      if (c < nchunk) {
        const f32x4 v = src[c];
        ((f32x4 *)lds_x)[c] = v;
        s = (v.x + v.y) + (v.z + v.w);
      }
      s = lane_group_sum<8>(s);
      if (c < nchunk && (c & 7) == 0) lds_sum[c >> 3] = s;
    }
  }
}

// Per-lane constants of the 6-bit scale/min decode for sub-blocks 2c, 2c+1.
struct ScaleDecode {
  uint32_t lo_sc0, lo_m0, lo_sc1, lo_m1;  // offsets of the low field
  uint32_t lo_w;                          // width of the low field (6 or 4)
  uint32_t hi_sc0, hi_m0, hi_sc1, hi_m1;  // offsets of the high 2 bits
  uint32_t hi_w;                          // 0 (j < 4) or 2 (j >= 4)
  bool upper;                             // sub-blocks 4..7
};

__device__ __forceinline__ ScaleDecode make_scale_decode(int c) {
  ScaleDecode s;
  const int j0 = 2 * c;
  s.upper = j0 >= 4;
  if (!s.upper) {
    s.lo_sc0 = 8 * j0; s.lo_m0 = 8 * j0; s.lo_sc1 = 8 * j0 + 8; s.lo_m1 = 8 * j0 + 8;
    s.lo_w = 6; s.hi_w = 0;
    s.hi_sc0 = s.hi_m0 = s.hi_sc1 = s.hi_m1 = 0;
  } else {
    const int jj = j0 - 4;
    s.lo_sc0 = 8 * jj; s.lo_m0 = 8 * jj + 4; s.lo_sc1 = 8 * jj + 8; s.lo_m1 = 8 * jj + 12;
    s.lo_w = 4; s.hi_w = 2;
    s.hi_sc0 = 8 * jj + 6; s.hi_m0 = 8 * jj + 6; s.hi_sc1 = 8 * jj + 14; s.hi_m1 = 8 * jj + 14;
  }
  return s;
}

// S0 = packed bytes 0..3, S1 = 4..7, S2 = 8..11. j < 4: sc from S0, m from
// S1 (6 bits). j >= 4: low 4 bits from S2 (sc low nibble, m high nibble),
// high 2 bits from the top of S0 (sc) / S1 (m).
__device__ __forceinline__ void decode_scales(const ScaleDecode &s, uint32_t S0, uint32_t S1,
                                              uint32_t S2, uint32_t &sc0, uint32_t &m0,
                                              uint32_t &sc1, uint32_t &m1) {
  const uint32_t Asc = s.upper ? S2 : S0;
  const uint32_t Am = s.upper ? S2 : S1;
  sc0 = bfe(Asc, s.lo_sc0, s.lo_w) | (bfe(S0, s.hi_sc0, s.hi_w) << 4);
  m0 = bfe(Am, s.lo_m0, s.lo_w) | (bfe(S1, s.hi_m0, s.hi_w) << 4);
  sc1 = bfe(Asc, s.lo_sc1, s.lo_w) | (bfe(S0, s.hi_sc1, s.hi_w) << 4);
  m1 = bfe(Am, s.lo_m1, s.lo_w) | (bfe(S1, s.hi_m1, s.hi_w) << 4);
}

// Q5 = true reads Q5_K blocks (176 B): the same header, a 32-byte high-bit
// plane at byte 16 whose bit j of byte l is the fifth bit of weight l of
// sub-block j, and the Q4_K code bytes at byte 48. Each lane also loads the
// whole high-bit plane and merges bits 2c and 2c+1 into its code bytes.
template <bool XBF16, int MT, bool Q5>
__global__ __launch_bounds__(GV_THREADS) void q4k_gemv_kernel(
    const uint8_t *__restrict__ w, const void *__restrict__ x, float *__restrict__ y, int N,
    int K, int ldy, int rows_q, int rows_rem, int max_wg_blocks) {
  constexpr int BB = Q5 ? Q5K_BYTES : Q4K_BYTES;  // bytes per super-block
  constexpr int QOFF = Q5 ? 48 : 16;              // code bytes

  extern __shared__ uint32_t lds[];
  uint32_t *lds_x = lds;
  float *lds_sum = (float *)(lds + (XBF16 ? MT * K / 2 : MT * K));
  float *lds_part = lds_sum + MT * (K / 32);  // [MT][max_wg_blocks]

  const int nb = K / QK;
  const int bid = blockIdx.x;
  const int r0 = bid * rows_q + min(bid, rows_rem);
  const int r1 = r0 + rows_q + (bid < rows_rem ? 1 : 0);
  const int64_t B0 = (int64_t)r0 * nb;
  const int nblk = (r1 - r0) * nb;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 2, c = lane & 3;
  const int wb0 = (int)(((int64_t)wave * nblk) / GV_WAVES);
  const int wb1 = (int)(((int64_t)(wave + 1) * nblk) / GV_WAVES);
  const int iters = (wb1 - wb0 + 15) >> 4;

  // block index (relative to B0) and column block of this lane, iteration 0
  int fb = wb0 + g;
  const uint8_t *fptr = w + (B0 + fb) * BB;
  const int64_t fstep = 16 * BB;

  u32x4 H[GV_PF], A[GV_PF], Bq[GV_PF];
  u32x4 Ha[Q5 ? GV_PF : 1], Hb[Q5 ? GV_PF : 1];  // Q5_K high-bit plane
#pragma unroll
  for (int p = 0; p < GV_PF; p++) {
    if (p < iters && fb + 16 * p < wb1) {
      const uint8_t *blk = fptr + p * fstep;
      H[p] = *(const u32x4 *)blk;
      A[p] = *(const u32x4 *)(blk + QOFF + 32 * c);
      Bq[p] = *(const u32x4 *)(blk + QOFF + 16 + 32 * c);
      if constexpr (Q5) {
        Ha[p] = *(const u32x4 *)(blk + 16);
        Hb[p] = *(const u32x4 *)(blk + 32);
      }
    }
  }

  stage_x<XBF16, MT>(x, K, lds_x, lds_sum);
  __syncthreads();

  const ScaleDecode sd = make_scale_decode(c);
  // Q4_K codes are nibbles picked straight from the code words; Q5_K codes
  // are first assembled into bytes (nibble | high bit << 4), then picked
  const uint32_t MASK = opaque(Q5 ? 0x00FF00FFu : 0x000F000Fu), MAGIC = opaque(0x43004300u);
  const int s16 = 16 % nb;
  int kb = fb % nb;  // column block of this lane's current block
  int cb = fb;       // current block (relative to B0)

  for (int it0 = 0; it0 < iters; it0 += GV_PF) {
#pragma unroll
    for (int p = 0; p < GV_PF; p++) {
      const int it = it0 + p;
      if (it < iters) {
        const bool valid = cb < wb1;
        float contrib[MT];
#pragma unroll
        for (int m = 0; m < MT; m++) contrib[m] = 0.f;
        if (valid) {
          const u32x4 hdr = H[p];
          const float d = half_bits_to_float(hdr.x);
          const float dmin = half_bits_to_float(hdr.x >> 16);
          uint32_t sc0, m0, sc1, m1;
          decode_scales(sd, hdr.y, hdr.z, hdr.w, sc0, m0, sc1, m1);
          const float a0 = d * (float)sc0, b0 = dmin * (float)m0;
          const float a1 = d * (float)sc1, b1 = dmin * (float)m1;
          const uint32_t q[8] = {A[p].x, A[p].y, A[p].z, A[p].w,
                                 Bq[p].x, Bq[p].y, Bq[p].z, Bq[p].w};
          // code words of sub-block 2c (lo) and 2c+1 (hi), positions 4i .. 4i+3:
          // Q4_K keeps the raw words (the nibble is picked with the mask or a
          // shift by 4); Q5_K builds bytes q = nibble | high bit << 4
          uint32_t lo[8], hi[8];
#pragma unroll
          for (int i = 0; i < 8; i++) {
            if constexpr (Q5) {
              const uint32_t hbits[8] = {Ha[p].x, Ha[p].y, Ha[p].z, Ha[p].w,
                                         Hb[p].x, Hb[p].y, Hb[p].z, Hb[p].w};
              const uint32_t hh = hbits[i] >> (2 * c);
              lo[i] = (q[i] & 0x0F0F0F0Fu) | ((hh << 4) & 0x10101010u);
              hi[i] = ((q[i] >> 4) & 0x0F0F0F0Fu) | ((hh << 3) & 0x10101010u);
            } else {
              lo[i] = q[i];
              hi[i] = q[i] >> 4;
            }
          }
          const int e0 = kb * QK + 64 * c;  // first x element of sub-block 2c
          if constexpr (XBF16) {
            const float c0 = fmaf(128.f, a0, b0), c1 = fmaf(128.f, a1, b1);
#pragma unroll
            for (int m = 0; m < MT; m++) {
              const u32x4 *xv = (const u32x4 *)(lds_x + (m * K + e0) / 2);
              const float2 xs = *(const float2 *)(lds_sum + m * (K / 32) + (e0 >> 5));
              float s0 = 0.f, s1 = 0.f;
#pragma unroll
              for (int i = 0; i < 4; i++) {
                const u32x4 x0 = xv[i];      // sub-block 2c, l = 8i .. 8i+7
                const u32x4 x1 = xv[4 + i];  // sub-block 2c+1
                const uint32_t qa = lo[2 * i], qb = lo[2 * i + 1];
                const uint32_t qa4 = hi[2 * i], qb4 = hi[2 * i + 1];
                s0 = dot2_bf16((qa & MASK) | MAGIC, x0.x, s0);
                s0 = dot2_bf16(((qa >> 8) & MASK) | MAGIC, x0.y, s0);
                s0 = dot2_bf16((qb & MASK) | MAGIC, x0.z, s0);
                s0 = dot2_bf16(((qb >> 8) & MASK) | MAGIC, x0.w, s0);
                s1 = dot2_bf16((qa4 & MASK) | MAGIC, x1.x, s1);
                s1 = dot2_bf16(((qa4 >> 8) & MASK) | MAGIC, x1.y, s1);
                s1 = dot2_bf16((qb4 & MASK) | MAGIC, x1.z, s1);
                s1 = dot2_bf16(((qb4 >> 8) & MASK) | MAGIC, x1.w, s1);
              }
              float r = a0 * s0;
              r = fmaf(-c0, xs.x, r);
              r = fmaf(a1, s1, r);
              r = fmaf(-c1, xs.y, r);
              contrib[m] = r;
            }
          } else {
#pragma unroll
            for (int m = 0; m < MT; m++) {
              const f32x4 *xv = (const f32x4 *)((const float *)lds_x + m * K + e0);
              const float2 xs = *(const float2 *)(lds_sum + m * (K / 32) + (e0 >> 5));
              float s0 = 0.f, s1 = 0.f;
#pragma unroll
              for (int i = 0; i < 8; i++) {
                const f32x4 x0 = xv[i];
                const f32x4 x1 = xv[8 + i];
                const uint32_t cl = Q5 ? lo[i] : lo[i] & 0x0F0F0F0Fu;
                const uint32_t ch = Q5 ? hi[i] : hi[i] & 0x0F0F0F0Fu;
                s0 = fmaf(x0.x, (float)(cl & 255u), s0);
                s0 = fmaf(x0.y, (float)((cl >> 8) & 255u), s0);
                s0 = fmaf(x0.z, (float)((cl >> 16) & 255u), s0);
                s0 = fmaf(x0.w, (float)(cl >> 24), s0);
                s1 = fmaf(x1.x, (float)(ch & 255u), s1);
                s1 = fmaf(x1.y, (float)((ch >> 8) & 255u), s1);
                s1 = fmaf(x1.z, (float)((ch >> 16) & 255u), s1);
                s1 = fmaf(x1.w, (float)(ch >> 24), s1);
              }
              float r = a0 * s0;
              r = fmaf(-b0, xs.x, r);
              r = fmaf(a1, s1, r);
              r = fmaf(-b1, xs.y, r);
              contrib[m] = r;
            }
          }
        }
        // refill this slot with the block GV_PF iterations ahead
        const int nfb = cb + 16 * GV_PF;
        if (it + GV_PF < iters && nfb < wb1) {
          const uint8_t *blk = fptr + (it + GV_PF) * fstep;
          H[p] = *(const u32x4 *)blk;
          A[p] = *(const u32x4 *)(blk + QOFF + 32 * c);
          Bq[p] = *(const u32x4 *)(blk + QOFF + 16 + 32 * c);
          if constexpr (Q5) {
            Ha[p] = *(const u32x4 *)(blk + 16);
            Hb[p] = *(const u32x4 *)(blk + 32);
          }
        }
        // sum the block's 4 lanes; one lane stores the block's contribution
#pragma unroll
        for (int m = 0; m < MT; m++) {
          float v = contrib[m];
          v = lane_group_sum<4>(v);
          if (valid && c == 0) lds_part[m * max_wg_blocks + cb] = v;
        }
        cb += 16;
        kb += s16;
        if (kb >= nb) kb -= nb;
      }
    }
  }
  __syncthreads();

  // y[row] = sum of the row's block contributions, in block order.
  const int nrows = r1 - r0;
  for (int t = threadIdx.x; t < MT * nrows; t += GV_THREADS) {
    const int m = t / nrows, r = t - m * nrows;
    const float *pp = lds_part + m * max_wg_blocks + r * nb;
    float s = 0.f;
    for (int k = 0; k < nb; k++) s += pp[k];
    y[(int64_t)m * ldy + r0 + r] = s;
  }
}


// ---------------------------------------------------------------------------
// M = 1, bf16 x: dense-span kernel (the decode hot path).
//
// A wave loads a span of 32 consecutive super-blocks (32 x 144 B = 4.5 KiB;
// Q5_K 32 x 176 B = 5.5 KiB) with 1-KiB wave loads of non-temporal 16-byte
// lane loads from a wave-uniform base (the last load partly re-reads the
// span's last 16 bytes), keeps the next span in flight in registers while it
// computes the current one, and moves each span through its own LDS buffer.
// Two lanes share a super-block there: lane 2i + h decodes code chunks 2h and
// 2h + 1 of block i (sub-blocks 4h .. 4h+3: the header once per 128 weights,
// the codes with one v_and_or_b32 per two codes, v_dot2_f32_bf16 against x),
// and the pair's two halves are added in a fixed order. Half-size spans keep
// the workgroup's first burst of weight loads small (x, loaded first, is ready
// sooner) and the last span's math short. Eight waves per workgroup, two per
// SIMD: once the memory queues are full a wave stalls at its next load, and
// its SIMD then runs the other wave's block math (one wave per SIMD with two
// spans in flight left the math and the stalls in series).
// x lives in LDS as 560-byte records per 256-element column block: 512 bytes
// of bf16 (groups of four stored as x0, x2, x1, x3), the eight 32-element sums,
// and 16 bytes of padding so that lanes reading consecutive column blocks hit
// distinct LDS banks.
// ---------------------------------------------------------------------------
constexpr int DN_SPAN = 32;  // blocks per span, two lanes per block
template <bool Q5>
constexpr int dn_block_bytes() { return Q5 ? Q5K_BYTES : Q4K_BYTES; }
template <bool Q5>
constexpr int dn_span_bytes() { return DN_SPAN * dn_block_bytes<Q5>(); }
// 1-KiB wave loads per span (5 for Q4_K, 6 for Q5_K) and the LDS buffer they fill
template <bool Q5>
constexpr int dn_span_chunks() { return (dn_span_bytes<Q5>() + 1023) / 1024; }
template <bool Q5>
constexpr int dn_span_buf() { return 1024 * dn_span_chunks<Q5>(); }
constexpr int DN_XREC = 560;                          // LDS bytes per x column block
constexpr int DN_TARGET_WGS = 256;      // workgroups per launch (one per CU)
constexpr int DN_MAX_WG_BLOCKS = 8192;
constexpr size_t DN_LDS_LIMIT = 160 * 1024;
constexpr int DN_WAVES = 8;  // waves per workgroup of the dense kernel

template <int NCH>
struct Span {
  u32x4 r[NCH];
};

// Loads are unconditional so the compiler can count outstanding loads and
// wait for exactly the span it needs (a load behind a branch forces it to wait
// for every load in flight).

// x staging in two phases: every x load is issued first (before any weight
// load, so waiting for x never waits for weights), then the chunks are
// permuted into their records and summed. XC 16-byte chunks per thread
// (K <= 8 * XC * threads); loads past the end re-read the last chunk.
template <int THREADS, int XC>
struct XStage {
  u32x4 v[XC];

  __device__ __forceinline__ void load(const uint16_t *__restrict__ x, int K) {
    const int nchunk = K / 8;
#pragma unroll
    for (int i = 0; i < XC; i++) {
      const int c = min(i * THREADS + (int)threadIdx.x, nchunk - 1);
      v[i] = ((const u32x4 *)x)[c];
    }
  }

  __device__ __forceinline__ void store(int K, uint8_t *xrec) const {
    const int nchunk = K / 8;  // 32 chunks per 256-element record
#pragma unroll
    for (int i = 0; i < XC; i++) {
      if (i * THREADS < nchunk) {  // uniform
        const int c = i * THREADS + threadIdx.x;
        const u32x4 e = v[i];
        u32x4 p;
        p.x = (e.x & 0xFFFFu) | (e.y << 16);
        p.y = (e.x >> 16) | (e.y & 0xFFFF0000u);
        p.z = (e.z & 0xFFFFu) | (e.w << 16);
        p.w = (e.z >> 16) | (e.w & 0xFFFF0000u);
        float s = bf16_bits_to_float(e.x) + bf16_bits_to_float(e.x >> 16) +
                  bf16_bits_to_float(e.y) + bf16_bits_to_float(e.y >> 16) +
                  bf16_bits_to_float(e.z) + bf16_bits_to_float(e.z >> 16) +
                  bf16_bits_to_float(e.w) + bf16_bits_to_float(e.w >> 16);
        s = lane_group_sum<4>(s);
        if (c < nchunk) {
          *(u32x4 *)(xrec + (c >> 5) * DN_XREC + (c & 31) * 16) = p;
          if ((c & 3) == 0) *(float *)(xrec + (c >> 5) * DN_XREC + 512 + 4 * ((c & 31) >> 2)) = s;
        }
      }
    }
  }
};

// Half h of sum_k x[k] * w(k) over one super-block held in LDS (blk), x
// record xr: code chunks 2h and 2h + 1, i.e. sub-blocks j = 4h .. 4h+3 (32
// weights each, 6-bit scale sc_j and min m_j):
//   sum_l x_l w_l = d sc_j sum_l x_l q_l - dmin m_j xs_j,  xs_j = sum_l x_l,
// so the half is d * sum_j sc_j t_j - dmin * sum_j m_j xs_j with integer-valued
// sc_j, m_j and t_j = sum_l x_l q_l. The code pairs enter v_dot2 as the bf16
// values 128 + q, so t_j's sum starts at -128 xs_j. The scale bytes are
// unpacked four at a time with word masks (h = 0: low 6 bits of bytes 0-3 and
// 4-7; h = 1: low/high nibble of bytes 8-11 and the top 2 bits of bytes 0-7).
// Q5_K (Q5): codes at 48 and the high-bit plane at 16; the code bytes are
// assembled (nibble | bit 2cc or 2cc+1 of the plane << 4), and v_perm_b32
// forms the bf16 pairs from them (MAGIC = 0x43434343 then).
template <bool Q5>
__device__ __forceinline__ float q4k_half_dot_bf16(const uint8_t *blk, const uint8_t *xr, int h,
                                                   uint32_t MASK, uint32_t MAGIC) {
  constexpr int QOFF = Q5 ? 48 : 16;
  const u32x4 hdr = *(const u32x4 *)blk;
  const float d = half_bits_to_float(hdr.x), dmin = half_bits_to_float(hdr.x >> 16);
  const f32x4 xs4 = *(const f32x4 *)(xr + 512 + 16 * h);
  const float xs[4] = {xs4.x, xs4.y, xs4.z, xs4.w};
  const uint32_t S0 = hdr.y, S1 = hdr.z, S2 = hdr.w;
  const uint32_t scw = h ? (S2 & 0x0F0F0F0Fu) | ((S0 >> 2) & 0x30303030u) : S0 & 0x3F3F3F3Fu;
  const uint32_t mw = h ? ((S2 >> 4) & 0x0F0F0F0Fu) | ((S1 >> 2) & 0x30303030u) : S1 & 0x3F3F3F3Fu;
  const float sc[4] = {(float)(scw & 255u), (float)((scw >> 8) & 255u),
                       (float)((scw >> 16) & 255u), (float)(scw >> 24)};
  const float mn[4] = {(float)(mw & 255u), (float)((mw >> 8) & 255u),
                       (float)((mw >> 16) & 255u), (float)(mw >> 24)};
  float tsum = 0.f, msum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; j++) msum = fmaf(mn[j], xs[j], msum);
#pragma unroll
  for (int c2 = 0; c2 < 2; c2++) {
    const int cc = 2 * h + c2;
    const u32x4 qa = *(const u32x4 *)(blk + QOFF + 32 * cc);
    const u32x4 qb = *(const u32x4 *)(blk + QOFF + 16 + 32 * cc);
    const uint32_t q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    // code words of sub-blocks 2cc (lo) and 2cc+1 (hi), positions 4i .. 4i+3
    uint32_t lo[8], hi[8];
    if constexpr (Q5) {
      const u32x4 ha = *(const u32x4 *)(blk + 16), hb = *(const u32x4 *)(blk + 32);
      const uint32_t hbits[8] = {ha.x, ha.y, ha.z, ha.w, hb.x, hb.y, hb.z, hb.w};
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t hhb = hbits[i] >> (2 * cc);
        lo[i] = (q[i] & 0x0F0F0F0Fu) | ((hhb << 4) & 0x10101010u);
        hi[i] = ((q[i] >> 4) & 0x0F0F0F0Fu) | ((hhb << 3) & 0x10101010u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        lo[i] = q[i];
        hi[i] = q[i] >> 4;
      }
    }
    const u32x4 *xv0 = (const u32x4 *)(xr + 128 * cc);
    const u32x4 *xv1 = (const u32x4 *)(xr + 128 * cc + 64);
    float s0 = -128.f * xs[2 * c2], s1 = -128.f * xs[2 * c2 + 1];
#pragma unroll
    for (int t = 0; t < 4; t++) {
      const u32x4 x0 = xv0[t], x1 = xv1[t];
      const uint32_t qd0 = lo[2 * t], qd1 = lo[2 * t + 1];
      const uint32_t qd04 = hi[2 * t], qd14 = hi[2 * t + 1];
      if constexpr (Q5) {
        // whole code bytes: v_perm_b32 picks bytes (0, 2) or (1, 3) and sets
        // the high byte of each half to 0x43 (MAGIC holds 0x43 in every byte)
        s0 = dot2_bf16(__builtin_amdgcn_perm(MAGIC, qd0, 0x04020400u), x0.x, s0);
        s0 = dot2_bf16(__builtin_amdgcn_perm(MAGIC, qd0, 0x04030401u), x0.y, s0);
        s0 = dot2_bf16(__builtin_amdgcn_perm(MAGIC, qd1, 0x04020400u), x0.z, s0);
        s0 = dot2_bf16(__builtin_amdgcn_perm(MAGIC, qd1, 0x04030401u), x0.w, s0);
        s1 = dot2_bf16(__builtin_amdgcn_perm(MAGIC, qd04, 0x04020400u), x1.x, s1);
        s1 = dot2_bf16(__builtin_amdgcn_perm(MAGIC, qd04, 0x04030401u), x1.y, s1);
        s1 = dot2_bf16(__builtin_amdgcn_perm(MAGIC, qd14, 0x04020400u), x1.z, s1);
        s1 = dot2_bf16(__builtin_amdgcn_perm(MAGIC, qd14, 0x04030401u), x1.w, s1);
      } else {
        s0 = dot2_bf16((qd0 & MASK) | MAGIC, x0.x, s0);
        s0 = dot2_bf16(((qd0 >> 8) & MASK) | MAGIC, x0.y, s0);
        s0 = dot2_bf16((qd1 & MASK) | MAGIC, x0.z, s0);
        s0 = dot2_bf16(((qd1 >> 8) & MASK) | MAGIC, x0.w, s0);
        s1 = dot2_bf16((qd04 & MASK) | MAGIC, x1.x, s1);
        s1 = dot2_bf16(((qd04 >> 8) & MASK) | MAGIC, x1.y, s1);
        s1 = dot2_bf16((qd14 & MASK) | MAGIC, x1.z, s1);
        s1 = dot2_bf16(((qd14 >> 8) & MASK) | MAGIC, x1.w, s1);
      }
    }
    tsum = fmaf(sc[2 * c2], s0, tsum);
    tsum = fmaf(sc[2 * c2 + 1], s1, tsum);
    // keep each sub-block pair's LDS reads next to its math
    __builtin_amdgcn_sched_barrier(0);
  }
  return d * tsum - dmin * msum;
}

// WAVES waves per workgroup. Each wave holds one span in registers while it
// computes the previous one from its LDS buffer. Spans are handed out in order
// from a workgroup counter, so a wave whose data arrived late takes fewer
// spans and the waves finish together. nb_magic = ceil(2^32 / nb) gives the
// column block of block b as b - nb * umulhi(b, nb_magic), exact while
// b * nb < 2^32 (b < 8192 + nb here).
template <int WAVES, int XC, bool Q5>
__global__ __launch_bounds__(WAVES * WAVE) void q4k_gemv_m1_kernel(
    const uint8_t *__restrict__ w, const uint16_t *__restrict__ x, float *__restrict__ y,
    int K, int rows_q, int rows_rem, uint32_t nb_magic) {
  constexpr int DN_THREADS = WAVES * WAVE;
  constexpr int BB = dn_block_bytes<Q5>();
  constexpr int DN_SPAN_BYTES = dn_span_bytes<Q5>();
  constexpr int NCH = dn_span_chunks<Q5>();
  constexpr int SPAN_BUF = dn_span_buf<Q5>();
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int next_span;
  const int nb = K / QK;
  uint8_t *spanbuf = smem;                            // [waves][NCH KiB]
  uint8_t *xrec = smem + WAVES * SPAN_BUF;            // [nb][560]
  float *part = (float *)(xrec + nb * DN_XREC);       // [blocks of this workgroup]

  const int bid = blockIdx.x;
  const int r0 = bid * rows_q + min(bid, rows_rem);
  const int r1 = r0 + rows_q + (bid < rows_rem ? 1 : 0);
  const int nblk = (r1 - r0) * nb;
  const int nspan = (nblk + DN_SPAN - 1) / DN_SPAN;
  const uint8_t *wbase = w + (int64_t)r0 * nb * BB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // span indices stay scalar
  const int nfull = nblk / DN_SPAN;  // spans before nfull are full

  // A span index past the end loads the last span again (its bytes are
  // already on their way), so every wave issues the same NCH loads in every
  // iteration and the compiler can wait for exactly the span it needs. The
  // span base is wave-uniform; lane offsets past the end of a span (the last
  // 1-KiB load of every span, and a partial span's tail) are clamped to its
  // last 16 bytes.
  auto issue = [&](Span<NCH> &r, int sidx) {
    const int si = min(sidx, nspan - 1);
    const uint8_t *base = wbase + (int64_t)si * DN_SPAN_BYTES;
    const int lim = (si < nfull ? DN_SPAN_BYTES : (nblk - DN_SPAN * si) * BB) - 16;
#pragma unroll
    for (int j = 0; j < NCH; j++) {
      const uint32_t off = (uint32_t)min(1024 * j + 16 * lane, lim);
      r.r[j] = __builtin_nontemporal_load((const u32x4 *)(base + off));
    }
  };
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&next_span, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };

  XStage<DN_THREADS, XC> xst;
  xst.load(x, K);
  if (threadIdx.x == 0) next_span = WAVES;
  int sidx = wave;
  // x loads, the first span, then the x records: x does not wait behind the
  // workgroup's whole initial burst of weight loads
  Span<NCH> R;
  issue(R, sidx);
  xst.store(K, xrec);
  __syncthreads();

  const uint32_t MASK = opaque(0x000F000Fu), MAGIC = opaque(Q5 ? 0x43434343u : 0x43004300u);
  uint8_t *mybuf = spanbuf + wave * SPAN_BUF;
  const int h = lane & 1;
  while (sidx < nspan) {
    const int cur = sidx;
    // every chunk is stored: the buffer holds NCH KiB, and what lies past the
    // span's bytes is never read
#pragma unroll
    for (int j = 0; j < NCH; j++) *(u32x4 *)(mybuf + 1024 * j + 16 * lane) = R.r[j];
    // refill right away: the next span is in flight during the math
    sidx = grab();
    issue(R, sidx);
    const int b = DN_SPAN * cur + (lane >> 1);
    float r = 0.f;
    if (b < nblk) {
      const uint32_t kb = nb == 1 ? 0u : (uint32_t)b - (uint32_t)nb * __umulhi((uint32_t)b, nb_magic);
      r = q4k_half_dot_bf16<Q5>(mybuf + BB * (lane >> 1), xrec + kb * DN_XREC, h, MASK, MAGIC);
    }
    r += __shfl_xor(r, 1, WAVE);  // half 0 + half 1 (the same sum on both lanes)
    if (b < nblk && h == 0) part[b] = r;
  }
  __syncthreads();

  const int nrows = r1 - r0;
  if ((nb & 3) == 0) {
    // A row's partials start 16-byte aligned: four running sums over 16-byte
    // reads keep the LDS reads independent (one latency, not one per block).
    for (int t = threadIdx.x; t < nrows; t += DN_THREADS) {
      const f32x4 *pp = (const f32x4 *)(part + t * nb);
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      for (int k = 0; k < nb / 4; k++) {
        const f32x4 v = pp[k];
        a0 += v.x;
        a1 += v.y;
        a2 += v.z;
        a3 += v.w;
      }
      y[r0 + t] = (a0 + a1) + (a2 + a3);
    }
  } else {
    for (int t = threadIdx.x; t < nrows; t += DN_THREADS) {
      const float *pp = part + t * nb;
      float sacc = 0.f;
      for (int k = 0; k < nb; k++) sacc += pp[k];
      y[r0 + t] = sacc;
    }
  }
}

// Launch geometry of the dense kernel, or false if its LDS does not fit.
template <int DN_WAVES, bool Q5>
bool dense_plan(int64_t N, int64_t K, int64_t &nwg, int &rows_q, int &rows_rem, size_t &lds) {
  const int64_t nb = K / QK;
  nwg = DN_TARGET_WGS;
  const int64_t need = (N * nb + DN_MAX_WG_BLOCKS - 1) / DN_MAX_WG_BLOCKS;
  if (need > nwg) nwg = need;
  if (nwg > N) nwg = N;
  rows_q = (int)(N / nwg);
  rows_rem = (int)(N % nwg);
  const int64_t max_blocks = (rows_q + (rows_rem ? 1 : 0)) * nb;
  lds = (size_t)DN_WAVES * dn_span_buf<Q5>() + (size_t)nb * DN_XREC + (size_t)max_blocks * 4;
  return lds <= DN_LDS_LIMIT && K / 8 <= (int64_t)16 * DN_WAVES * WAVE;
}

// x chunks per thread for K (the smallest instantiated count that covers it).
template <int DN_WAVES, int XC, bool Q5>
void launch_dense(const void *w, const void *x, float *y, int64_t K, int64_t nwg, int rows_q,
                  int rows_rem, size_t lds, hipStream_t s) {
  auto kern = q4k_gemv_m1_kernel<DN_WAVES, XC, Q5>;
  (void)hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
  const uint64_t nb = (uint64_t)(K / QK);
  const uint32_t nb_magic = (uint32_t)((((uint64_t)1 << 32) + nb - 1) / nb);  // unused for nb = 1
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(DN_WAVES * WAVE), lds, s,
                     (const uint8_t *)w, (const uint16_t *)x, y, (int)K, rows_q, rows_rem,
                     nb_magic);
}

template <bool XBF16, int MT, bool Q5>
void launch_chunk(const void *w, const void *x, float *y, int64_t N, int64_t K, int64_t ldy,
                  hipStream_t s) {
  const int64_t nb = K / QK;
  // Enough workgroups to fill the device; more when a workgroup's block slots
  // (MT floats per block) would exceed their LDS budget: 32 KiB, or what the
  // 160 KiB of LDS leave beside x, less one row's slots (a workgroup holds up
  // to one row more than the average).
  int64_t nwg = GV_TARGET_WGS;
  const size_t x_lds = (size_t)MT * K * (XBF16 ? 2 : 4) + (size_t)MT * (K / 32) * 4;
  const size_t part_budget = x_lds < 128 * 1024 ? 32768 : 160 * 1024 - x_lds;
  const int64_t cap = (int64_t)(part_budget / (4 * MT)) - nb;  // blocks per workgroup
  const int64_t need = (N * nb + cap - 1) / cap;
  if (need > nwg) nwg = need;
  if (nwg > N) nwg = N;
  const int rows_q = (int)(N / nwg), rows_rem = (int)(N % nwg);
  const int max_wg_blocks = (int)((rows_q + (rows_rem ? 1 : 0)) * nb);
  const size_t lds = x_lds + (size_t)MT * max_wg_blocks * 4;
  auto kern = q4k_gemv_kernel<XBF16, MT, Q5>;
  if (lds > 65536)
    (void)hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(GV_THREADS), lds, s, (const uint8_t *)w, x,
                     y, (int)N, (int)K, (int)ldy, rows_q, rows_rem, max_wg_blocks);
}

// Rows of x in chunks of MT (1, 2, 4 or 8) per launch of the general kernel,
// as many as fit a 64 KiB LDS budget for x (several workgroups per compute
// unit); when that budget holds a single row but more rows remain (long K),
// up to 148 KiB (one workgroup per unit, fewer passes over the weights).
template <bool Q5>
void launch_general(const void *w, const void *x, bool x_bf16, float *y, int64_t M, int64_t N,
                    int64_t K, hipStream_t s) {
  const size_t per_row = (size_t)K * (x_bf16 ? 2 : 4) + (size_t)(K / 32) * 4;
  const size_t elt = x_bf16 ? 2 : 4;
  int64_t m0 = 0;
  while (m0 < M) {
    const int64_t rem = M - m0;
    int mt = 8;
    while (mt > 1 && (mt > rem || (size_t)mt * per_row > 65536)) mt >>= 1;
    if (mt == 1 && rem > 1) {
      mt = 8;
      while (mt > 1 && (mt > rem || (size_t)mt * per_row > 148 * 1024)) mt >>= 1;
    }
    const void *xm = (const char *)x + (size_t)m0 * K * elt;
    float *ym = y + m0 * N;
    if (x_bf16) {
      switch (mt) {
        case 8: launch_chunk<true, 8, Q5>(w, xm, ym, N, K, N, s); break;
        case 4: launch_chunk<true, 4, Q5>(w, xm, ym, N, K, N, s); break;
        case 2: launch_chunk<true, 2, Q5>(w, xm, ym, N, K, N, s); break;
        default: launch_chunk<true, 1, Q5>(w, xm, ym, N, K, N, s); break;
      }
    } else {
      switch (mt) {
        case 8: launch_chunk<false, 8, Q5>(w, xm, ym, N, K, N, s); break;
        case 4: launch_chunk<false, 4, Q5>(w, xm, ym, N, K, N, s); break;
        case 2: launch_chunk<false, 2, Q5>(w, xm, ym, N, K, N, s); break;
        default: launch_chunk<false, 1, Q5>(w, xm, ym, N, K, N, s); break;
      }
    }
    m0 += mt;
  }
}

}  // namespace

// M = 1 with bf16 x runs the dense-span kernel whenever its LDS plan fits
// (K up to about 26K for Q4_K); other cases (fp32 x, M > 1, longer K) process
// rows of x in chunks of MT (1, 2, 4 or 8) per launch of the general kernel,
// as many as fit a 64 KiB LDS budget for x.
// The dense-span kernel for M = 1 with bf16 x, or false if its LDS plan does
// not fit.
template <bool Q5>
bool try_dense(const void *w, const void *x, float *y, int64_t N, int64_t K, hipStream_t s) {
  int64_t nwg;
  int rows_q, rows_rem;
  size_t lds;
  if (!dense_plan<DN_WAVES, Q5>(N, K, nwg, rows_q, rows_rem, lds)) return false;
  const int64_t per_thread = (K / 8 + DN_WAVES * WAVE - 1) / (DN_WAVES * WAVE);
  if (per_thread <= 2)
    launch_dense<DN_WAVES, 2, Q5>(w, x, y, K, nwg, rows_q, rows_rem, lds, s);
  else if (per_thread <= 3)
    launch_dense<DN_WAVES, 3, Q5>(w, x, y, K, nwg, rows_q, rows_rem, lds, s);
  else if (per_thread <= 5)
    launch_dense<DN_WAVES, 5, Q5>(w, x, y, K, nwg, rows_q, rows_rem, lds, s);
  else if (per_thread <= 8)
    launch_dense<DN_WAVES, 8, Q5>(w, x, y, K, nwg, rows_q, rows_rem, lds, s);
  else
    launch_dense<DN_WAVES, 16, Q5>(w, x, y, K, nwg, rows_q, rows_rem, lds, s);
  return true;
}

// With bf16 x and M >= 2 the matrix-core GEMV (weights rounded to bf16 once,
// every x row on the matrix cores): the general kernel spends M dot products
// per weight and at M = 8 took 182 us for the gate+up shape.
void launch_q4k_gemv(const void *w, const void *x, bool x_bf16, float *y, int64_t M,
                     int64_t N, int64_t K, hipStream_t s) {
  if (M == 1 && x_bf16 && try_dense<false>(w, x, y, N, K, s)) return;
  if (M >= 2 && x_bf16 && ((uintptr_t)w & 15) == 0) {
    launch_q4k_mfma_gemv(w, (const uint16_t *)x, y, M, N, K, false, s);
    return;
  }
  launch_general<false>(w, x, x_bf16, y, M, N, K, s);
}

// Q5_K: the same choice between the dense-span, matrix-core and general kernels.
void launch_q5k_gemv(const void *w, const void *x, bool x_bf16, float *y, int64_t M,
                     int64_t N, int64_t K, hipStream_t s) {
  if (M == 1 && x_bf16 && try_dense<true>(w, x, y, N, K, s)) return;
  if (M >= 2 && x_bf16 && ((uintptr_t)w & 15) == 0) {
    launch_q4k_mfma_gemv(w, (const uint16_t *)x, y, M, N, K, true, s);
    return;
  }
  launch_general<true>(w, x, x_bf16, y, M, N, K, s);
}

}  // namespace qdm
