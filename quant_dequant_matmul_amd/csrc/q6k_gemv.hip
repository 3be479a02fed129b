// Q6_K GEMV: y[m][n] = sum_k x[m][k] * w(n, k) for M in 1..16 (VALU path).
//
// Q6_K is the output-head / mixed tensor type of a Q4_K_M file (hipEngine
// README, "GGUF Support", payload table). Weight i of a 210-byte block, with
// h = i/128, g = (i%128)/32, l = i%32: low nibble from QL[64h + 32(g%2) + l]
// (high half when g >= 2), high pair from bits 2g..2g+1 of QH[32h + l],
// w = d * scale[i/16] * (q - 32).
//
// Mapping (wave64): a lane owns half h = c/2 and the 16 positions
// l0 = 16(c%2) .. l0+15 of a block, i.e. 64 weights (4 groups g of 16, each
// one sub-block with its own scale). 4 lanes per block; rows split across the
// 16 lane-groups of a wave as in the Q4_K GEMV (G = gcd(K/256, 16) groups per
// row, R = 16/G rows per wave).
//
// Alignment: blocks are 210 bytes, so a block starts at an even offset; all
// field offsets a lane reads (64h + l0, 64h + 32 + l0, 128 + 32h + l0, 192 +
// 8h, 208) are even too. Each field is read as 4-byte-aligned dwords covering
// it and shifted down by 0 or 2 bytes with v_alignbyte.
//
// bf16 x: codes become exact bf16 values 128 + q (q < 64 fits the 7-bit
// mantissa at exponent 7), summed with v_dot2_f32_bf16 against x pairs
// (l, l+2) / (l+1, l+3) (x staged in LDS with groups of four permuted), then
//   sum_l x_l (q_l - 32) = s - 160 * sum_l x_l.
#include "common.h"
#include "launch.h"
#include "q4k_tile.h"  // pack_bf16

namespace qdm {

namespace {


template <bool XBF16, int MT, int THREADS>
__device__ __forceinline__ void q6_stage_x(const void *__restrict__ x, int K, uint32_t *lds_x,
                                           float *lds_sum) {
  const int tid = threadIdx.x;
  if constexpr (XBF16) {
    const int nchunk = MT * K / 8;  // 8 bf16 per chunk, 2 chunks per 16-sum
    const u32x4 *src = (const u32x4 *)x;
    for (int base = 0; base < nchunk; base += THREADS) {
      const int c = base + tid;
      float s = 0.f;
      if (c < nchunk) {
        const u32x4 v = src[c];
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
      s = lane_group_sum<2>(s);
      if (c < nchunk && (c & 1) == 0) lds_sum[c >> 1] = s;
    }
  } else {
    const int nchunk = MT * K / 4;  // 4 fp32 per chunk, 4 chunks per 16-sum
    const f32x4 *src = (const f32x4 *)x;
    for (int base = 0; base < nchunk; base += THREADS) {
      const int c = base + tid;
      float s = 0.f;
      if (c < nchunk) {
        const f32x4 v = src[c];
        ((f32x4 *)lds_x)[c] = v;
        s = (v.x + v.y) + (v.z + v.w);
      }
      s = lane_group_sum<4>(s);
      if (c < nchunk && (c & 3) == 0) lds_sum[c >> 2] = s;
    }
  }
}

// 4-byte-aligned dword loads (the compiler must not assume more alignment).
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// 16 bytes starting at an even byte offset `off` from the 16-aligned base:
// five aligned dwords [off & ~3, (off & ~3) + 20), shifted down by (off & 2)
// bytes. Callers keep off + 18 inside the block.
__device__ __forceinline__ u32x4 load16_even(const uint8_t *__restrict__ base, int64_t off) {
  const int64_t a = off & ~(int64_t)3;
  const u32x4 lo = *(const u32x4_a4 *)(base + a);
  const uint32_t hi = *(const uint32_t *)(base + a + 16);
  const uint32_t sh = (uint32_t)(off & 2);
  u32x4 r;
  r.x = __builtin_amdgcn_alignbyte(lo.y, lo.x, sh);
  r.y = __builtin_amdgcn_alignbyte(lo.z, lo.y, sh);
  r.z = __builtin_amdgcn_alignbyte(lo.w, lo.z, sh);
  r.w = __builtin_amdgcn_alignbyte(hi, lo.w, sh);
  return r;
}

// 4 bytes at an even offset: the dwords holding its first and last byte
// (the same dword when off is 4-aligned). Never reads past off + 6.
__device__ __forceinline__ uint32_t load4_even(const uint8_t *__restrict__ base, int64_t off) {
  const uint32_t lo = *(const uint32_t *)(base + (off & ~(int64_t)3));
  const uint32_t hi = *(const uint32_t *)(base + ((off + 2) & ~(int64_t)3));
  return __builtin_amdgcn_alignbyte(hi, lo, (uint32_t)(off & 2));
}

struct Q6Lane {
  u32x4 qa, qb, qh;  // QL[64h+l0..], QL[64h+32+l0..], QH[32h+l0..]
  uint32_t s0, s1;   // scale bytes 8h .. 8h+7
  uint32_t dbits;    // fp16 d in the low half
};

__device__ __forceinline__ Q6Lane q6_load(const uint8_t *__restrict__ w, int64_t blk_off, int h,
                                          int l0) {
  Q6Lane L;
  L.qa = load16_even(w, blk_off + 64 * h + l0);
  L.qb = load16_even(w, blk_off + 64 * h + 32 + l0);
  L.qh = load16_even(w, blk_off + 128 + 32 * h + l0);
  L.s0 = load4_even(w, blk_off + 192 + 8 * h);
  L.s1 = load4_even(w, blk_off + 196 + 8 * h);
  L.dbits = *(const uint16_t *)(w + blk_off + 208);  // 2-aligned; the last field
  return L;
}

// d * scale for the four 16-weight groups gq of lane (h, l0): group gq is
// sub-block 8h + 2gq + l0/16, byte 2gq + l0/16 of the 8 scale bytes s0|s1.
__device__ __forceinline__ void q6_dsc(const Q6Lane &L, int l0, float (&dsc)[4]) {
  const float d = half_bits_to_float(L.dbits);
  const int sb = l0 >> 4;
#pragma unroll
  for (int gq = 0; gq < 4; gq++) {
    const int bi = 2 * gq + sb;
    const uint32_t word = bi < 4 ? L.s0 : L.s1;
    dsc[gq] = d * (float)(int8_t)(uint8_t)(word >> (8 * (bi & 3)));
  }
}

// The 64 codes of lane (h, l0) as bf16 pairs 128 + q (exact: q < 64 fits the
// 7-bit mantissa at exponent 7): pr[gq][2k + e] for group gq, code dword k,
// e = 0 -> (l, l+2), 1 -> (l+1, l+3). Four 6-bit codes are first assembled as
// bytes (low nibble from ql | two bits of qh << 4); v_perm_b32 then picks
// bytes (0, 2) or (1, 3) and sets the high byte of each half to 0x43.
__device__ __forceinline__ void q6_pairs(const Q6Lane &L, uint32_t (&pr)[4][8]) {
  const uint32_t qa[4] = {L.qa.x, L.qa.y, L.qa.z, L.qa.w};
  const uint32_t qb[4] = {L.qb.x, L.qb.y, L.qb.z, L.qb.w};
  const uint32_t qh[4] = {L.qh.x, L.qh.y, L.qh.z, L.qh.w};
  const uint32_t EXP = 0x43434343u;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const uint32_t a = qa[k], b = qb[k], hh = qh[k];
    const uint32_t c[4] = {(a & 0x0F0F0F0Fu) | ((hh << 4) & 0x30303030u),
                           (b & 0x0F0F0F0Fu) | ((hh << 2) & 0x30303030u),
                           ((a >> 4) & 0x0F0F0F0Fu) | (hh & 0x30303030u),
                           ((b >> 4) & 0x0F0F0F0Fu) | ((hh >> 2) & 0x30303030u)};
#pragma unroll
    for (int g = 0; g < 4; g++) {
      pr[g][2 * k + 0] = __builtin_amdgcn_perm(EXP, c[g], 0x04020400u);
      pr[g][2 * k + 1] = __builtin_amdgcn_perm(EXP, c[g], 0x04030401u);
    }
  }
}

// One block's contribution for every row m of x: lane (h, l0)'s 64 weights
// against x staged in LDS, added to acc[m] (4 dot-product groups of 16, each
// scaled by its sub-block scale).
template <bool XBF16, int MT>
__device__ __forceinline__ void q6_block(const Q6Lane &L, const uint32_t *lds_x,
                                         const float *lds_sum, int K, int kb, int h, int l0,
                                         float (&acc)[MT]) {
  float dsc[4];
  q6_dsc(L, l0, dsc);
  const uint32_t qa[4] = {L.qa.x, L.qa.y, L.qa.z, L.qa.w};
  const uint32_t qb[4] = {L.qb.x, L.qb.y, L.qb.z, L.qb.w};
  const uint32_t qh[4] = {L.qh.x, L.qh.y, L.qh.z, L.qh.w};
  if constexpr (XBF16) {
    uint32_t pr[4][8];
    q6_pairs(L, pr);
#pragma unroll
    for (int m = 0; m < MT; m++) {
      float r = acc[m];
#pragma unroll
      for (int gq = 0; gq < 4; gq++) {
        const int e0 = m * K + kb * QK + 128 * h + 32 * gq + l0;  // first x element
        const u32x4 *xv = (const u32x4 *)(lds_x + e0 / 2);
        const float xs = lds_sum[e0 / 16];
        const u32x4 x0 = xv[0], x1 = xv[1];  // l0..l0+7, l0+8..l0+15
        float s = 0.f;
        s = dot2_bf16(pr[gq][0], x0.x, s);
        s = dot2_bf16(pr[gq][1], x0.y, s);
        s = dot2_bf16(pr[gq][2], x0.z, s);
        s = dot2_bf16(pr[gq][3], x0.w, s);
        s = dot2_bf16(pr[gq][4], x1.x, s);
        s = dot2_bf16(pr[gq][5], x1.y, s);
        s = dot2_bf16(pr[gq][6], x1.z, s);
        s = dot2_bf16(pr[gq][7], x1.w, s);
        r = fmaf(dsc[gq], fmaf(-160.f, xs, s), r);
      }
      acc[m] = r;
    }
  } else {
#pragma unroll
    for (int m = 0; m < MT; m++) {
      float r = acc[m];
#pragma unroll
      for (int gq = 0; gq < 4; gq++) {
        const int e0 = m * K + kb * QK + 128 * h + 32 * gq + l0;
        const f32x4 *xv = (const f32x4 *)((const float *)lds_x + e0);
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const f32x4 xx = xv[k];
          const uint32_t src = (gq & 1) ? qb[k] : qa[k];
          const int nsh = (gq >> 1) * 4;
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const int lo = (int)((src >> (8 * e + nsh)) & 15u);
            const int hi = (int)((qh[k] >> (8 * e + 2 * gq)) & 3u);
            s = fmaf(xx[e], (float)((lo | (hi << 4)) - 32), s);
          }
        }
        r = fmaf(dsc[gq], s, r);
      }
      acc[m] = r;
    }
  }
}

// Each workgroup stages x once and then streams row groups blockIdx.x,
// blockIdx.x + gridDim.x, ... (a row group = R rows per wave). A wave walks
// its (row group, block iteration) pairs as one flat sequence with PF of them
// in flight, so loads run ahead across row-group boundaries. Loads are
// unconditional (indices clamped) so the waits are exact.
template <bool XBF16, int MT, int PF, int THREADS>
__global__ __launch_bounds__(THREADS) void q6k_gemv_kernel(
    const uint8_t *__restrict__ w, const void *__restrict__ x, float *__restrict__ y, int N,
    int K, int G, int ldy) {
  extern __shared__ uint32_t lds[];
  uint32_t *lds_x = lds;
  float *lds_sum = (float *)(lds + (XBF16 ? MT * K / 2 : MT * K));

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 2, c = lane & 3;
  const int h = c >> 1, l0 = 16 * (c & 1);
  const int R = 16 / G;
  const int gg = g % G;
  const int nb = K / QK;
  const int iters = nb / G;
  const int rows_rg = (THREADS / WAVE) * R;
  const int nrg = (N + rows_rg - 1) / rows_rg;
  const int mine = (int)blockIdx.x < nrg ? (nrg - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int64_t nf = (int64_t)mine * iters;  // this wave's (row group, iteration) pairs
  auto row_of = [&](int64_t f) {
    const int j = (int)(f / iters);
    return ((int)blockIdx.x + j * (int)gridDim.x) * rows_rg + wave * R + g / G;
  };
  auto blk_off = [&](int64_t f) {
    const int64_t fc = f < nf ? f : nf - 1;
    const int it = (int)(fc % iters);
    const int row = min(row_of(fc), N - 1);
    return ((int64_t)row * nb + it * G + gg) * Q6K_BYTES;
  };

  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; m++) acc[m] = 0.f;

  Q6Lane buf[PF];
  if (nf > 0) {
#pragma unroll
    for (int p = 0; p < PF; p++) buf[p] = q6_load(w, blk_off(p), h, l0);
  }

  q6_stage_x<XBF16, MT, THREADS>(x, K, lds_x, lds_sum);
  __syncthreads();

  for (int64_t f0 = 0; f0 < nf; f0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; p++) {
      const int64_t f = f0 + p;
      if (f < nf) {
        const int it = (int)(f % iters);
        const int kb = it * G + gg;
        const Q6Lane L = buf[p];
        buf[p] = q6_load(w, blk_off(f + PF), h, l0);
        q6_block<XBF16, MT>(L, lds_x, lds_sum, K, kb, h, l0, acc);
        if (it == iters - 1) {  // uniform: the row group ends, store its rows
          const int row = row_of(f);
#pragma unroll
          for (int m = 0; m < MT; m++) {
            const float v = group_sum(acc[m], 4 * G);
            if (row < N && (lane & (4 * G - 1)) == 0) y[(int64_t)m * ldy + row] = v;
            acc[m] = 0.f;
          }
        }
      }
    }
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
  // the 8-row chunk keeps all of x for 8 rows in LDS (one workgroup per
  // compute unit), so it runs 8 waves per workgroup for latency hiding
  constexpr int THREADS = MT == 8 ? 512 : 256;
  const int64_t rows_per_rg = (int64_t)(THREADS / WAVE) * R;
  const int64_t nrg = (N + rows_per_rg - 1) / rows_per_rg;
  const size_t lds = (size_t)MT * K * (XBF16 ? 2 : 4) + (size_t)MT * (K / 16) * 4;
  // as many workgroups as stay resident (x is staged once per workgroup)
  int64_t per_cu = (int64_t)(160 * 1024 / (lds + 1024));
  if (per_cu < 1) per_cu = 1;
  if (per_cu > 4) per_cu = 4;
  const int64_t want = 256 * per_cu;
  const unsigned grid = (unsigned)(nrg < want ? nrg : want);
  constexpr int PF = 2;
  auto kern = q6k_gemv_kernel<XBF16, MT, PF, THREADS>;
  if (lds > 65536) (void)hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(THREADS), lds, s, (const uint8_t *)w, x, y,
                     (int)N, (int)K, G, (int)ldy);
}

// ---------------------------------------------------------------------------
// M >= 2 with bf16 x: matrix cores. At M = 8 the VALU path spends 8 dot
// products per weight and is bound by them; here every weight is decoded to
// bf16 once, w = d * scale * (q - 32) (exact in fp32, then rounded to nearest
// even), and v_mfma_f32_16x16x32_bf16 multiplies it with all M rows of x.
// A wave streams tiles of 16 weight rows. Lane (s, r) = (lane / 16, lane % 16)
// loads, for row r of the tile, the same 64-weight slice (h, l0) = (s / 2,
// 16 (s % 2)) of each super-block that a VALU lane loads, so a wave's loads
// cover 16 rows x whole super-blocks. Step (g, e) of a super-block, g = 0..3,
// e = 0..1, gives the lane's weights at positions 128h + 32g + l0 + 8e + j,
// j = 0..7, as the A operand; the B operand is x row (lane % 16) at the same
// positions, from LDS (rows of x past M repeat row M - 1; their outputs are
// not stored; the rows are staged with LDS-direct copies). The matrix core
// pairs A and B by (lane / 16, j), so any K order that both sides share gives
// the same contraction.
// Work split: workgroup b owns an even share of the 16-row tiles, and its
// waves split the share's (tile, super-block) items into equal contiguous
// ranges, so every wave streams the same number of super-blocks. A tile cut
// by a range boundary is finished by the wave that holds its first
// super-block: the waves that continue it publish their portion (the first
// portion of their range) in LDS, and the first wave adds those portions in
// wave order before it stores. Loads run Q6M_PF items ahead.
// Staged loads: a lane's slice is scattered over one row, so every load
// instruction touches all 16 rows and each line of an item is requested by
// several instructions. When staging, the wave instead loads the item's 16 row
// blocks as consecutive 16-byte chunks (consecutive lanes read consecutive
// bytes of a row), writes them to its own LDS rows and reads the slices back
// from there; the next item's loads go out as soon as the chunks are written.
// ---------------------------------------------------------------------------
constexpr int Q6_MFMA_MIN_M = 2;  // smallest M (bf16 x) that takes the matrix-core kernel
constexpr int Q6M_PF = 2;         // super-blocks in flight per wave
constexpr size_t Q6M_FLAGS = 256;  // flag words, padded
constexpr int Q6M_SPIN_LIMIT = 1 << 24;

__host__ __device__ constexpr size_t q6m_head_bytes(int waves) {
  return (size_t)waves * WAVE * sizeof(f32x4) + Q6M_FLAGS;
}

// LDS for M rows of x with K columns: rows of K + 8 bf16 (16 bytes of padding)
// in whole KiB, the unit of one wave's LDS-direct copy.
__host__ __device__ constexpr size_t kq_x_bytes(int64_t M, int64_t K) {
  return (size_t)((M * (K / 8 + 1) + WAVE - 1) / WAVE) * 1024;
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ __forceinline__ uint32_t q6m_codes(uint32_t ql, uint32_t qh, int g) {
  // four 6-bit codes of group g as bytes: low nibble (g < 2) or high nibble of
  // ql, and bits 2g, 2g + 1 of qh as bits 4, 5
  const uint32_t lo = g < 2 ? ql : ql >> 4;
  const uint32_t hi = g == 0 ? qh << 4 : g == 1 ? qh << 2 : g == 2 ? qh : qh >> 2;
  return (lo & 0x0F0F0F0Fu) | (hi & 0x30303030u);
}

// A lane's slice (h, l0) of one super-block as loaded: aligned dwords only,
// so the loads stay in flight until the slice is decoded. The super-block
// starts at an even byte offset; every field the slice reads starts at the
// same offset mod 4, so one shift (0 or 2 bytes) realigns them all.
struct Q6Raw {
  u32x4 qa, qb, qh;           // 16 B from the dword holding QL[64h+l0], QL[64h+32+l0], QH[32h+l0]
  uint32_t qa4, qb4, qh4;     // the dword after each
  uint32_t sc0, sc1, sc2;     // dwords covering scale bytes 8h .. 8h+7
  uint32_t dbits, sh;
};

__device__ __forceinline__ Q6Raw q6_load_raw(const uint8_t *__restrict__ w, int64_t blk_off,
                                             int h, int l0) {
  Q6Raw R;
  const int64_t a = blk_off & ~(int64_t)3;
  const int64_t fa = a + 64 * h + l0, fb = fa + 32, fh = a + 128 + 32 * h + l0;
  R.qa = *(const u32x4_a4 *)(w + fa);
  R.qa4 = *(const uint32_t *)(w + fa + 16);
  R.qb = *(const u32x4_a4 *)(w + fb);
  R.qb4 = *(const uint32_t *)(w + fb + 16);
  R.qh = *(const u32x4_a4 *)(w + fh);
  R.qh4 = *(const uint32_t *)(w + fh + 16);
  // scale bytes [so, so + 8): dwords at so & ~3, +4, and (so + 6) & ~3, which
  // is the third dword when so is 2 mod 4 and a re-read of the second
  // otherwise (never past the super-block)
  const int64_t so = blk_off + 192 + 8 * h;
  typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
  const u32x2_a4 s01 = *(const u32x2_a4 *)(w + (so & ~(int64_t)3));
  R.sc0 = s01.x;
  R.sc1 = s01.y;
  R.sc2 = *(const uint32_t *)(w + ((so + 6) & ~(int64_t)3));
  R.dbits = *(const uint16_t *)(w + blk_off + 208);
  R.sh = (uint32_t)(blk_off & 2);
  return R;
}

__device__ __forceinline__ Q6Lane q6_finish(const Q6Raw &R) {
  Q6Lane L;
  auto al = [&](const u32x4 &v, uint32_t n) {
    return u32x4{__builtin_amdgcn_alignbyte(v.y, v.x, R.sh), __builtin_amdgcn_alignbyte(v.z, v.y, R.sh),
                 __builtin_amdgcn_alignbyte(v.w, v.z, R.sh), __builtin_amdgcn_alignbyte(n, v.w, R.sh)};
  };
  L.qa = al(R.qa, R.qa4);
  L.qb = al(R.qb, R.qb4);
  L.qh = al(R.qh, R.qh4);
  L.s0 = __builtin_amdgcn_alignbyte(R.sc1, R.sc0, R.sh);
  L.s1 = __builtin_amdgcn_alignbyte(R.sc2, R.sc1, R.sh);
  L.dbits = R.dbits;
  return L;
}

// Format policies of the matrix-core GEMV. Lane group s = lane / 16 owns a
// 64-weight slice of every super-block; step t = 0..7 of an item gives the
// lane's A operand, 8 weights decoded to bf16, and the B operand is x at the
// same 8 positions of the super-block (any order shared by A and B gives the
// same contraction). Weights are exact in fp32 and rounded to bf16 (nearest
// even) once.
//
// Q6_K: slice (h, l0) = (s / 2, 16 (s % 2)); step t = 2g + e covers positions
// 128h + 32g + l0 + 8e + j, group g's scale.
struct MfQ6 {
  static constexpr int BYTES = Q6K_BYTES;
  // staged copy: a row's block is copied as the 14 aligned 16-byte chunks that
  // cover it (it starts at an even offset), rows 240 bytes apart in LDS
  static constexpr bool STAGE_OK = true;
  static constexpr int ONE_CU_WAVES = 12;
  static constexpr int STAGE_CPR = 14, STAGE_RS = 240;
  static constexpr bool STAGE_SHIFT = true;
  typedef Q6Raw Raw;
  __device__ static Raw load(const uint8_t *__restrict__ w, int64_t blk_off, int s) {
    return q6_load_raw(w, blk_off, s >> 1, 16 * (s & 1));
  }
  __device__ static void mfma(const Raw &R, int s, const uint16_t *xk, f32x4 (&acc2)[2]) {
    const int h = s >> 1, l0 = 16 * (s & 1);
    const Q6Lane L = q6_finish(R);
    const float d = half_bits_to_float(L.dbits);
    const uint32_t qa[4] = {L.qa.x, L.qa.y, L.qa.z, L.qa.w};
    const uint32_t qb[4] = {L.qb.x, L.qb.y, L.qb.z, L.qb.w};
    const uint32_t qh[4] = {L.qh.x, L.qh.y, L.qh.z, L.qh.w};
    const uint16_t *xs = xk + 128 * h + l0;
#pragma unroll
    for (int g = 0; g < 4; g++) {
      // scale of sub-block 8h + 2g + l0/16: byte 2g + l0/16 of s0|s1
      const int bi = 2 * g + (l0 >> 4);
      const uint32_t word = bi < 4 ? L.s0 : L.s1;
      const float ds = d * (float)(int8_t)(uint8_t)(word >> (8 * (bi & 3)));
      const float nds = -32.f * ds;
#pragma unroll
      for (int e = 0; e < 2; e++) {
        uint32_t pk[4];
#pragma unroll
        for (int k2 = 0; k2 < 2; k2++) {
          const int k = 2 * e + k2;
          const uint32_t c4 = q6m_codes((g & 1) ? qb[k] : qa[k], qh[k], g);
          pk[2 * k2] = pack_bf16(fmaf((float)(c4 & 255u), ds, nds),
                                 fmaf((float)((c4 >> 8) & 255u), ds, nds));
          pk[2 * k2 + 1] = pack_bf16(fmaf((float)((c4 >> 16) & 255u), ds, nds),
                                     fmaf((float)(c4 >> 24), ds, nds));
        }
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
        const bf16x8 bv = *(const bf16x8 *)(xs + 32 * g + 8 * e);
        acc2[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc2[e], 0, 0, 0);
      }
    }
  }
};

// Q4_K / Q5_K (Q5): slice s is code chunk s, i.e. sub-blocks 2s (low nibbles)
// and 2s + 1 (high nibbles); step t covers positions 64s + 8t + j, sub-block
// 2s + t / 4. w = q * (d sc) - dmin m with one rounding (fma: the product is
// exact). Q5_K adds bit 2s (or 2s + 1) of high-plane byte l as bit 4 of q.
template <bool Q5>
struct MfQ4 {
  static constexpr int BYTES = Q5 ? Q5K_BYTES : Q4K_BYTES;
  static constexpr int QOFF = Q5 ? 48 : 16;
  static constexpr bool STAGE_OK = true;
  static constexpr int ONE_CU_WAVES = 12;
  static constexpr int STAGE_CPR = BYTES / 16, STAGE_RS = BYTES;
  static constexpr bool STAGE_SHIFT = false;
  struct Raw {
    u32x4 hdr, qa, qb;
    u32x4 ha[Q5 ? 1 : 0], hb[Q5 ? 1 : 0];
  };
  __device__ static Raw load(const uint8_t *__restrict__ w, int64_t blk_off, int s) {
    Raw R;
    const uint8_t *b = w + blk_off;  // 16-byte aligned
    R.hdr = *(const u32x4 *)b;
    R.qa = *(const u32x4 *)(b + QOFF + 32 * s);
    R.qb = *(const u32x4 *)(b + QOFF + 32 * s + 16);
    if constexpr (Q5) {
      R.ha[0] = *(const u32x4 *)(b + 16);
      R.hb[0] = *(const u32x4 *)(b + 32);
    }
    return R;
  }
  __device__ static void mfma(const Raw &R, int s, const uint16_t *xk, f32x4 (&acc2)[2]) {
    const float d = half_bits_to_float(R.hdr.x), dmin = half_bits_to_float(R.hdr.x >> 16);
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min(R.hdr.y, R.hdr.z, R.hdr.w, 2 * s, sc0, m0);
    q4k_scale_min(R.hdr.y, R.hdr.z, R.hdr.w, 2 * s + 1, sc1, m1);
    const float a0 = d * (float)sc0, nb0 = -(dmin * (float)m0);  // exact products
    const float a1 = d * (float)sc1, nb1 = -(dmin * (float)m1);
    // Q4_K: a code byte (0..15) read as fp8 e4m3 is exactly q * 2^-9, so
    // v_cvt_pk_f32_fp8 converts two codes at once and the scale carries 2^9:
    // fma(q * 2^-9, a * 2^9, -b) is the same single rounding as fma(q, a, -b)
    const uint32_t q[8] = {R.qa.x, R.qa.y, R.qa.z, R.qa.w, R.qb.x, R.qb.y, R.qb.z, R.qb.w};
    const uint16_t *xs = xk + 64 * s;
#pragma unroll
    for (int t = 0; t < 8; t++) {
      const bool hi = t >= 4;
      const float a = hi ? a1 : a0, nb = hi ? nb1 : nb0;
      uint32_t pk[4];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int k = 2 * (t & 3) + u;  // code dword: weights 4k .. 4k+3 of the sub-block
        uint32_t c = (hi ? q[k] >> 4 : q[k]) & 0x0F0F0F0Fu;
        if constexpr (Q5) {
          const uint32_t hp[8] = {R.ha[0].x, R.ha[0].y, R.ha[0].z, R.ha[0].w,
                                  R.hb[0].x, R.hb[0].y, R.hb[0].z, R.hb[0].w};
          c |= ((hp[k] >> (2 * s + (hi ? 1 : 0))) << 4) & 0x10101010u;
        }
        if constexpr (Q5) {
          pk[2 * u] = pack_bf16(fmaf((float)(c & 255u), a, nb), fmaf((float)((c >> 8) & 255u), a, nb));
          pk[2 * u + 1] = pack_bf16(fmaf((float)((c >> 16) & 255u), a, nb),
                                    fmaf((float)(c >> 24), a, nb));
        } else {
          const float a9 = a * 512.f;
          const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
          const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, true);
          pk[2 * u] = pack_bf16(fmaf(f01[0], a9, nb), fmaf(f01[1], a9, nb));
          pk[2 * u + 1] = pack_bf16(fmaf(f23[0], a9, nb), fmaf(f23[1], a9, nb));
        }
      }
      const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
      const bf16x8 bv = *(const bf16x8 *)(xs + 8 * t);
      acc2[t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc2[t & 1], 0, 0, 0);
    }
  }
};

// Q8_0: a "super-block" is 8 blocks of 34 bytes (272 B, 256 weights; rows
// start 16-byte aligned when K % 256 == 0). Lane group s takes blocks 2s and
// 2s + 1 (68 bytes from a 4-byte aligned offset); step t covers positions
// 64s + 8t + j, block 2s + t/4, codes 8 (t % 4) .. +7 of it. w = d * q, exact
// in fp32, then rounded to bf16.
struct MfQ8 {
  static constexpr int BYTES = 8 * Q80_BYTES;
  // direct loads: the staged copy (five chunks per lane) spills registers at
  // 12 waves per compute unit and measured slower
  static constexpr bool STAGE_OK = false;
  // 8 waves when one workgroup fills a CU (each item is 4.25 KiB; with 12
  // waves more loads queue: K=5120 N=7168 M=8 14.5 -> 13.3 us)
  static constexpr int ONE_CU_WAVES = 8;
  static constexpr int STAGE_CPR = BYTES / 16, STAGE_RS = BYTES;
  static constexpr bool STAGE_SHIFT = false;
  struct Raw {
    u32x4 v[4];
    uint32_t t;
  };
  __device__ static Raw load(const uint8_t *__restrict__ w, int64_t blk_off, int s) {
    typedef uint32_t u32x4_a4l __attribute__((ext_vector_type(4), aligned(4)));
    Raw R;
    const uint8_t *b = w + blk_off + 68 * s;
#pragma unroll
    for (int i = 0; i < 4; i++) R.v[i] = *(const u32x4_a4l *)(b + 16 * i);
    R.t = *(const uint32_t *)(b + 64);
    return R;
  }
  __device__ static void mfma(const Raw &R, int s, const uint16_t *xk, f32x4 (&acc2)[2]) {
    uint32_t D[17];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      D[4 * i] = R.v[i].x;
      D[4 * i + 1] = R.v[i].y;
      D[4 * i + 2] = R.v[i].z;
      D[4 * i + 3] = R.v[i].w;
    }
    D[16] = R.t;
    // block 2s: d in bytes 0-1, codes from byte 2 (2 bytes into a dword);
    // block 2s + 1: d in bytes 34-35 (dword 8, upper half), codes from byte 36
    const float d0 = half_bits_to_float(D[0]), d1 = half_bits_to_float(D[8] >> 16);
    const uint16_t *xs = xk + 64 * s;
#pragma unroll
    for (int t = 0; t < 8; t++) {
      const bool hi = t >= 4;
      const float d = hi ? d1 : d0;
      uint32_t c[2];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int k = 2 * (t & 3) + u;  // code dword k of the block
        c[u] = hi ? D[9 + k] : __builtin_amdgcn_alignbyte(D[k + 1], D[k], 2);
      }
      uint32_t pk[4];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        pk[2 * u] = pack_bf16(d * (float)(int8_t)(c[u] & 255u),
                              d * (float)(int8_t)((c[u] >> 8) & 255u));
        pk[2 * u + 1] = pack_bf16(d * (float)(int8_t)((c[u] >> 16) & 255u),
                                  d * (float)(int8_t)(c[u] >> 24));
      }
      const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
      const bf16x8 bv = *(const bf16x8 *)(xs + 8 * t);
      acc2[t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc2[t & 1], 0, 0, 0);
    }
  }
};

// One launch covers the K columns [256 kb0, 256 kb0 + K) of rows that are
// ldk columns long (x rows too: x points at column 256 kb0 of row 0); with
// accumulate set it adds its sums to y (column chunks of a long K).
// Staged copy of one item: NCI 16-byte chunks per lane cover 16 rows of
// STAGE_CPR chunks each (the last load instruction repeats the final chunk in
// its spare lanes).
template <class Fmt>
struct KqStage {
  static constexpr int CPR = Fmt::STAGE_CPR, RS = Fmt::STAGE_RS;
  static constexpr int NCI = (16 * CPR + WAVE - 1) / WAVE;
  static constexpr size_t WAVE_BYTES = (size_t)16 * RS;  // LDS per wave
  struct Raw {
    u32x4 c[NCI];
  };
};

template <int THREADS, class Fmt, bool STAGE>
__global__ __launch_bounds__(THREADS) void kq_mfma_kernel(const uint8_t *__restrict__ w,
                                                          const uint16_t *__restrict__ x,
                                                          float *__restrict__ y, int M, int N,
                                                          int K, int xs, int ldk, int kb0,
                                                          int accumulate) {
  constexpr int WAVES = THREADS / WAVE;
  typedef KqStage<Fmt> St;
  constexpr size_t STAGE_BYTES = STAGE ? WAVES * St::WAVE_BYTES : 0;
  extern __shared__ __attribute__((aligned(16))) uint8_t q6m_smem[];
  f32x4 *part = (f32x4 *)q6m_smem;                                   // [WAVES][64]
  int *flag = (int *)(q6m_smem + (size_t)WAVES * WAVE * sizeof(f32x4));  // [WAVES]
  uint8_t *stage = q6m_smem + q6m_head_bytes(WAVES);                // [WAVES][16][RS]
  uint16_t *xl = (uint16_t *)(stage + STAGE_BYTES);                  // [M][xs] bf16
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform ranges
  const int nb = K / QK, nbt = ldk / QK;
  const int tiles = (N + 15) / 16;
  const int tq = tiles / (int)gridDim.x, tr = tiles % (int)gridDim.x;
  const int bid = blockIdx.x;
  const int t0 = bid * tq + min(bid, tr);
  const int items = (tq + (bid < tr ? 1 : 0)) * nb;  // >= nb: every workgroup has a tile
  auto start_of = [&](int v) { return (int)((int64_t)items * v / WAVES); };
  const int i0 = start_of(wave), i1 = start_of(wave + 1);
  const int s = lane >> 4, r = lane & 15;

  if (tid < WAVES) flag[tid] = 0;
  // staged copy, per lane: chunk k is chunk sj[k] of tile row srow[k], kept
  // at byte sdst[k] of the wave's LDS rows
  int srow[St::NCI], sj[St::NCI];
  uint32_t sdst[St::NCI];
#pragma unroll
  for (int k = 0; k < St::NCI; k++) {
    const int c = min(lane + WAVE * k, 16 * St::CPR - 1);
    srow[k] = c / St::CPR;
    sj[k] = c - srow[k] * St::CPR;
    sdst[k] = (uint32_t)(srow[k] * St::RS + 16 * sj[k]);
  }
  uint8_t *sbuf = stage + (size_t)wave * St::WAVE_BYTES;
  // The compute and load streams walk (tile, block) positions with counters
  // (no division per item). Addresses are a wave-uniform tile base plus 32-bit
  // lane offsets (16 rows of one tile).
  struct Pos {
    int tl, b;
  };
  auto pos_of = [&](int i) {
    const int tl = i / nb;
    return Pos{tl, i - tl * nb};
  };
  auto step = [&](Pos &p) {
    if (++p.b == nb) {
      p.b = 0;
      p.tl++;
    }
  };
  const uint32_t rowbytes = (uint32_t)nbt * Fmt::BYTES;
  auto load_at = [&](Pos p) {
    const uint8_t *tb = w + (int64_t)(t0 + p.tl) * 16 * rowbytes;  // 16-byte aligned
    const int lastr = N - 1 - (t0 + p.tl) * 16;                     // rows past N repeat it
    const uint32_t boff = (uint32_t)(kb0 + p.b) * Fmt::BYTES;
    if constexpr (STAGE) {
      // a row's chunks start at its block rounded down to 16 bytes; for Q6_K
      // the last chunk may run up to 14 bytes past the block, which stays
      // inside the tensor when its size is a multiple of 16 bytes
      typename St::Raw R;
#pragma unroll
      for (int k = 0; k < St::NCI; k++) {
        uint32_t g = (uint32_t)min(srow[k], lastr) * rowbytes + boff;
        if constexpr (Fmt::STAGE_SHIFT) g &= ~15u;
        R.c[k] = *(const u32x4 *)(tb + g + 16 * sj[k]);
      }
      return R;
    } else {
      return Fmt::load(tb, (int64_t)((uint32_t)min(r, lastr) * rowbytes + boff), s);
    }
  };
  typedef decltype(load_at(Pos{0, 0})) Buf;
  // load stream: items from i0 on; past the range it reloads the range's last
  // item (a valid dummy)
  int lnext = i0;
  Pos lp = pos_of(i0);
  const Pos lend = pos_of(max(i1 - 1, 0));
  auto load_next = [&]() {
    const Pos p = lnext < i1 ? lp : lend;
    lnext++;
    step(lp);
    return load_at(p);
  };
  // stage x rows [0, M) with row stride xs (K + 8 elements: rows start 4 banks
  // apart) by LDS-direct copies, all in flight at once: 16-byte slot sl of the
  // staged rows is chunk sl % (K/8 + 1) of row sl / (K/8 + 1) (a row's padding
  // slot repeats its last chunk), one KiB of consecutive slots per wave copy;
  // the last copy's slots past the rows repeat the last one (the LDS holds
  // whole KiB). The weight loads of the first items follow; the barrier waits
  // for every copy.
  {
    const int spr = K / 8 + 1, nslot = M * spr, ncopy = (nslot + WAVE - 1) / WAVE;
    for (int i = wave; i < ncopy; i += WAVES) {  // uniform
      const int sl = min(i * WAVE + lane, nslot - 1);
      const int m = sl / spr;
      const int j = min(sl - m * spr, spr - 2);
      __builtin_amdgcn_global_load_lds((const void *)(x + (int64_t)m * ldk + 8 * j),
                                       (lds_ptr_t)((uint8_t *)xl + 1024 * i), 16, 0, 0);
    }
  }
  Buf buf[Q6M_PF];
#pragma unroll
  for (int p = 0; p < Q6M_PF; p++) buf[p] = load_next();
  __syncthreads();

  const uint16_t *xb = xl + min(r, M - 1) * xs;
  // two accumulators (steps e = 0 and e = 1) halve the MFMA dependency chain
  f32x4 acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // one item: decode the slice, 8 MFMAs; at the end of this wave's portion of
  // a tile, publish it or complete and store the tile
  Pos cp = pos_of(i0);  // compute stream
  auto item = [&](int ii, Buf &slot, bool reload) {
    const int tl = cp.tl, b = cp.b;
    step(cp);
    if constexpr (STAGE) {
      // only this wave uses its LDS rows, and a wave's LDS accesses run in
      // order: the previous item's slice reads are done before these writes
#pragma unroll
      for (int k = 0; k < St::NCI; k++) *(u32x4 *)(sbuf + sdst[k]) = slot.c[k];
      if (reload) slot = load_next();
      uint32_t sh = 0;  // where the lane's row block starts in its LDS row
      if constexpr (Fmt::STAGE_SHIFT) {
        const int row = min((t0 + tl) * 16 + r, N - 1);
        sh = ((uint32_t)row * (uint32_t)nbt + (uint32_t)(kb0 + b)) * (uint32_t)Fmt::BYTES & 15u;
      }
      const typename Fmt::Raw R = Fmt::load(sbuf, (int64_t)(r * St::RS + sh), s);
      Fmt::mfma(R, s, xb + b * QK, acc2);
    } else {
      Fmt::mfma(slot, s, xb + b * QK, acc2);
      if (reload) slot = load_next();
    }

    if (b == nb - 1 || ii == i1 - 1) {  // end of this wave's portion of a tile
      f32x4 acc = acc2[0] + acc2[1];
      const int tstart = tl * nb;
      if (tstart < i0) {
        // the tile began in an earlier wave's range: publish the portion
        part[wave * WAVE + lane] = acc;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __hip_atomic_store(&flag[wave], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        // the rest of the tile is the first portion of the next ranges
        for (int v = wave + 1; v < WAVES && start_of(v) < tstart + nb; v++) {
          if (start_of(v) == start_of(v + 1)) continue;  // empty range
          int spins = 0;
          while (__hip_atomic_load(&flag[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) ==
                     0 &&
                 spins < Q6M_SPIN_LIMIT) {
            __builtin_amdgcn_s_sleep(1);
            spins++;
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
          const f32x4 o = part[v * WAVE + lane];
          acc += o;
          if (spins >= Q6M_SPIN_LIMIT) acc = f32x4{NAN, NAN, NAN, NAN};
        }
        // lane holds column m = lane % 16 and rows 4 (lane / 16) + q of the tile
        const int m = lane & 15;
        if (m < M) {
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int n = (t0 + tl) * 16 + 4 * s + q;
            if (n < N) {
              float *yo = y + (int64_t)m * N + n;
              *yo = accumulate ? *yo + acc[q] : acc[q];
            }
          }
        }
      }
      acc2[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc2[1] = acc2[0];
    }
  };
  // whole groups of Q6M_PF items run with every load unconditional, so each
  // wait is for exactly one item's loads; then the last partial group
  int i = i0;
  for (; i + Q6M_PF <= i1; i += Q6M_PF) {
#pragma unroll
    for (int p = 0; p < Q6M_PF; p++) item(i + p, buf[p], true);
  }
#pragma unroll
  for (int p = 0; p < Q6M_PF; p++)
    if (i + p < i1) item(i + p, buf[p], false);
}

template <int THREADS, class Fmt, bool STAGE>
void launch_q6_mfma(const void *w, const uint16_t *x, float *y, int mc, int64_t N, int64_t K,
                    int64_t ldk, int64_t kb0, bool accumulate, size_t lds, int per_cu,
                    hipStream_t s) {
  const int64_t tiles = (N + 15) / 16;
  int64_t grid = 256 * per_cu;
  if (grid > tiles) grid = tiles;  // every workgroup owns at least one tile
  auto kern = kq_mfma_kernel<THREADS, Fmt, STAGE>;
  (void)hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(THREADS), lds, s, (const uint8_t *)w, x,
                     y, mc, (int)N, (int)K, (int)(K + 8), (int)ldk, (int)kb0, accumulate ? 1 : 0);
}

// All M rows of x in every launch; when their padded LDS copy would not fit,
// K is split into equal chunks of whole super-blocks, each launch streaming
// only its columns of the weights and adding into y after the first (the
// weights are read once; splitting M instead would read them per split).
// 12 waves per compute unit (3 per SIMD, as many as the registers allow):
// 3 workgroups of 4 waves, 2 of 6, or 1 of 12, whichever LDS allows (1 of 8
// when K is split into chunks, and for Q8_0).
// Staged loads take one set of 16 LDS rows per wave (12 per compute unit);
// they are used unless they would need more K chunks, or (Q6_K, whose staged
// chunks may run up to 14 bytes past a block) the tensor's size is not a
// multiple of 16 bytes.
template <class Fmt, bool STAGE>
void launch_kq_mfma_x(const void *w, const uint16_t *x, float *y, int64_t M, int64_t N,
                      int64_t K, int64_t nch, hipStream_t s) {
  constexpr size_t LDS_CU = 160 * 1024, SLACK = 512;  // SLACK: static LDS, rounding
  constexpr size_t SW = STAGE ? KqStage<Fmt>::WAVE_BYTES : 0;
  const int64_t units = K / QK;
  int64_t kb0 = 0;
  for (int64_t c = 0; c < nch; c++) {
    const int64_t kc = (units / nch + (c < units % nch ? 1 : 0)) * QK;
    const size_t xb = kq_x_bytes(M, kc);
    const uint16_t *xm = x + kb0 * QK;
    const int mc = (int)M;
    const bool acc = c > 0;
    const size_t l4 = xb + q6m_head_bytes(4) + 4 * SW, l6 = xb + q6m_head_bytes(6) + 6 * SW;
    const size_t l8 = xb + q6m_head_bytes(8) + 8 * SW, l12 = xb + q6m_head_bytes(12) + 12 * SW;
    if (3 * (l4 + SLACK) <= LDS_CU)
      launch_q6_mfma<256, Fmt, STAGE>(w, xm, y, mc, N, kc, K, kb0, acc, l4, 3, s);
    else if (2 * (l6 + SLACK) <= LDS_CU)
      launch_q6_mfma<384, Fmt, STAGE>(w, xm, y, mc, N, kc, K, kb0, acc, l6, 2, s);
    else if (nch > 1 || Fmt::ONE_CU_WAVES == 8)
      // one workgroup per CU with 8 waves (2 per SIMD) rather than 12: faster
      // when K is split into chunks (Q5_K K=17408 N=5120 M=8: 38.0 -> 36.2 us)
      // and for the formats that ask for it
      launch_q6_mfma<512, Fmt, STAGE>(w, xm, y, mc, N, kc, K, kb0, acc, l8, 1, s);
    else
      launch_q6_mfma<768, Fmt, STAGE>(w, xm, y, mc, N, kc, K, kb0, acc, l12, 1, s);
    kb0 += kc / QK;
  }
}

template <class Fmt>
void launch_kq_mfma(const void *w, const uint16_t *x, float *y, int64_t M, int64_t N,
                    int64_t K, hipStream_t s) {
  constexpr size_t LDS_CU = 160 * 1024, SLACK = 512;
  const int64_t units = K / QK;
  auto chunks = [&](size_t x_cap) {
    int64_t n = 1;
    while (kq_x_bytes(M, (units + n - 1) / n * QK) > x_cap) n++;
    return n;
  };
  const size_t x_cap = LDS_CU - SLACK - q6m_head_bytes(16);
  const int64_t nch = chunks(x_cap);
  const int64_t nch_st = chunks(x_cap - 12 * KqStage<Fmt>::WAVE_BYTES);
  const bool fits = !Fmt::STAGE_SHIFT || (N * units) % 8 == 0;
  if constexpr (Fmt::STAGE_OK) {
    if (fits && nch_st == nch) {
      launch_kq_mfma_x<Fmt, true>(w, x, y, M, N, K, nch, s);
      return;
    }
  }
  launch_kq_mfma_x<Fmt, false>(w, x, y, M, N, K, nch, s);
}

// ---------------------------------------------------------------------------
// M = 1, bf16 x: dense-span kernel. A workgroup (one per compute unit) owns
// a balanced range of whole rows whose bytes start on a 16-byte boundary
// (rows are handed out in units of u = 8 / gcd(K/256, 8), so r0 * K/256 * 210
// is a multiple of 16). Its eight waves (two per SIMD: one wave's math runs
// while the other stalls on a full memory queue) take spans of 32 consecutive
// blocks (6720 bytes: six 1-KiB wave loads plus 576 bytes) from a workgroup
// counter, keep the next span in flight in registers while computing the
// current one from their own LDS buffer, where lanes 2i and 2i + 1 share
// block i (lane 2i + h takes its half h, 128 weights, and the two halves are
// added in a fixed order): two (half, 16-lane
// offset) quarters, each read as aligned dwords shifted by v_alignbyte, with
// the same pair arithmetic as the VALU path. x is staged once per workgroup as
// 592-byte records per 256 columns: 512 bytes of bf16 in (x0, x2, x1, x3)
// groups, the sixteen 16-column sums, and 16 bytes of padding (a stride of
// 148 dwords, so consecutive records start 20 banks apart).
// ---------------------------------------------------------------------------
constexpr int Q6D_SPAN = 32;                                    // blocks per span, 2 lanes each
constexpr int Q6D_SPAN_BYTES = Q6D_SPAN * Q6K_BYTES;            // 6720
constexpr int Q6D_NCH = (Q6D_SPAN_BYTES + 1023) / 1024;         // 7 loads per lane
constexpr int Q6D_SPAN_BUF = 1024 * Q6D_NCH;                    // LDS per wave
constexpr int Q6D_XREC = 592;
constexpr int Q6D_WAVES = 8;
constexpr int Q6D_THREADS = Q6D_WAVES * WAVE;
constexpr int Q6D_TARGET_WGS = 256;
constexpr size_t Q6D_LDS_LIMIT = 160 * 1024;

struct Q6Span {
  u32x4 r[Q6D_NCH];
};

// x staging: XC 8-element chunks per thread, all loaded before the first
// weight load and stored after it (storing waits for the x loads only).
template <int XC>
struct Q6XStage {
  u32x4 v[XC];

  __device__ __forceinline__ void load(const uint16_t *__restrict__ x, int K) {
    const int nchunk = K / 8;
#pragma unroll
    for (int i = 0; i < XC; i++)
      v[i] = ((const u32x4 *)x)[min(i * Q6D_THREADS + (int)threadIdx.x, nchunk - 1)];
  }

  __device__ __forceinline__ void store(int K, uint8_t *xrec) const {
    const int nchunk = K / 8;  // 32 chunks per record, 2 per 16-column sum
#pragma unroll
    for (int i = 0; i < XC; i++) {
      if (i * Q6D_THREADS < nchunk) {  // uniform
        const int c = i * Q6D_THREADS + threadIdx.x;
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
        s = lane_group_sum<2>(s);
        if (c < nchunk) {
          uint8_t *rec = xrec + (c >> 5) * Q6D_XREC;
          *(u32x4 *)(rec + 16 * (c & 31)) = p;
          if ((c & 1) == 0) *(float *)(rec + 512 + 4 * ((c & 31) >> 1)) = s;
        }
      }
    }
  }
};

// Quarter (h, l0) of a block against its x record xr (bf16 pairs).
__device__ __forceinline__ float q6_quarter_rec(const Q6Lane &L, const uint8_t *xr, int h,
                                                int l0) {
  float dsc[4];
  q6_dsc(L, l0, dsc);
  uint32_t pr[4][8];
  q6_pairs(L, pr);
  float r = 0.f;
#pragma unroll
  for (int gq = 0; gq < 4; gq++) {
    const int j0 = 128 * h + 32 * gq + l0;  // first column of the group in the record
    const u32x4 x0 = *(const u32x4 *)(xr + 2 * j0), x1 = *(const u32x4 *)(xr + 2 * j0 + 16);
    const float xs = *(const float *)(xr + 512 + 4 * (j0 >> 4));
    float sd = 0.f;
    sd = dot2_bf16(pr[gq][0], x0.x, sd);
    sd = dot2_bf16(pr[gq][1], x0.y, sd);
    sd = dot2_bf16(pr[gq][2], x0.z, sd);
    sd = dot2_bf16(pr[gq][3], x0.w, sd);
    sd = dot2_bf16(pr[gq][4], x1.x, sd);
    sd = dot2_bf16(pr[gq][5], x1.y, sd);
    sd = dot2_bf16(pr[gq][6], x1.z, sd);
    sd = dot2_bf16(pr[gq][7], x1.w, sd);
    r = fmaf(dsc[gq], fmaf(-160.f, xs, sd), r);
  }
  return r;
}

// floor(v / d) for 0 <= v < 2^16, 2 <= d < 2^16, magic = ceil(2^32 / d)
// (d = 1 has no 32-bit magic; callers handle it).
__device__ __forceinline__ int q6_div(int v, uint32_t magic) {
  return (int)__umulhi((uint32_t)v, magic);
}

template <int XC>
__global__ __launch_bounds__(Q6D_THREADS) void q6k_gemv_m1_kernel(
    const uint8_t *__restrict__ w, const uint16_t *__restrict__ x, float *__restrict__ y, int K,
    int unit, int units_q, int units_rem, int N, uint32_t nb_magic) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int next_span;
  const int nb = K / QK;
  uint8_t *spanbuf = smem;                                    // [waves][span bytes]
  uint8_t *xrec = smem + Q6D_WAVES * Q6D_SPAN_BUF;            // [nb][592]
  float *part = (float *)(xrec + nb * Q6D_XREC);              // [blocks of this workgroup]

  const int bid = blockIdx.x;
  const int r0 = unit * (bid * units_q + min(bid, units_rem));
  const int r1 = min(N, r0 + unit * (units_q + (bid < units_rem ? 1 : 0)));
  const int nblk = (r1 - r0) * nb;
  const int nspan = (nblk + Q6D_SPAN - 1) / Q6D_SPAN;
  const uint8_t *wbase = w + (int64_t)r0 * nb * Q6K_BYTES;   // 16-byte aligned
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Span si past the end reloads the last span; a chunk past the end of a
  // partial span re-reads its last 16 bytes (every span size is a multiple of
  // 16 bytes). Loads are unconditional so the waits count exactly; the span
  // base is wave-uniform and the lane offsets 32-bit.
  auto issue = [&](Q6Span &sp, int sidx) {
    const int si = __builtin_amdgcn_readfirstlane(min(sidx, nspan - 1));
    const int lim = min(Q6D_SPAN, nblk - Q6D_SPAN * si) * Q6K_BYTES - 16;
    const uint8_t *base = wbase + (int64_t)si * Q6D_SPAN_BYTES;
#pragma unroll
    for (int j = 0; j < Q6D_NCH; j++) {
      const uint32_t off = (uint32_t)min(1024 * j + 16 * lane, lim);
      sp.r[j] = __builtin_nontemporal_load((const u32x4 *)(base + off));
    }
  };
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&next_span, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };

  Q6XStage<XC> xst;
  xst.load(x, K);
  if (threadIdx.x == 0) next_span = Q6D_WAVES;
  int sidx = wave;
  Q6Span R;
  issue(R, sidx);
  xst.store(K, xrec);
  __syncthreads();

  uint8_t *mybuf = spanbuf + wave * Q6D_SPAN_BUF;
  const int h = lane & 1;
  while (sidx < nspan) {
    const int cur = sidx;
    // every chunk is stored: the buffer holds Q6D_NCH KiB, and what lies past
    // the span's bytes is never read
#pragma unroll
    for (int j = 0; j < Q6D_NCH; j++) *(u32x4 *)(mybuf + 1024 * j + 16 * lane) = R.r[j];
    // refill right away: the next span is in flight during the math
    sidx = grab();
    issue(R, sidx);
    const int b = Q6D_SPAN * cur + (lane >> 1);
    float r = 0.f;
    if (b < nblk) {
      const int kb = nb == 1 ? 0 : b - q6_div(b, nb_magic) * nb;
      const uint8_t *xr = xrec + kb * Q6D_XREC;
      const int off = Q6K_BYTES * (lane >> 1);
      r = q6_quarter_rec(q6_load(mybuf, off, h, 0), xr, h, 0);
      r += q6_quarter_rec(q6_load(mybuf, off, h, 16), xr, h, 16);
    }
    r += __shfl_xor(r, 1, WAVE);  // half 0 + half 1 (the same sum on both lanes)
    if (b < nblk && h == 0) part[b] = r;
  }
  __syncthreads();

  const int nrows = r1 - r0;
  for (int t = threadIdx.x; t < nrows; t += Q6D_THREADS) {
    const float *pp = part + t * nb;
    float sacc = 0.f;
    for (int k = 0; k < nb; k++) sacc += pp[k];
    y[r0 + t] = sacc;
  }
}

// Launch geometry of the dense kernel, or false if it does not apply: rows
// whose bytes start 16-byte aligned need N * K/256 to be a multiple of 8, and
// the spans, x records and one float per block of a workgroup must fit LDS.
bool q6_dense_plan(int64_t N, int64_t K, int &unit, int &units_q, int &units_rem,
                   int64_t &nwg, size_t &lds) {
  const int64_t nb = K / QK;
  int g = 8;
  while (nb % g) g >>= 1;  // gcd(nb, 8)
  unit = 8 / g;
  if (N % unit || N > INT32_MAX) return false;
  const int64_t units = N / unit;
  const size_t fixed = (size_t)Q6D_WAVES * Q6D_SPAN_BUF + (size_t)nb * Q6D_XREC;
  if (fixed + (size_t)unit * nb * 4 * 2 > Q6D_LDS_LIMIT) return false;
  const int64_t cap_units = (int64_t)((Q6D_LDS_LIMIT - fixed) / ((size_t)unit * nb * 4)) - 1;
  // one workgroup per compute unit, or a whole multiple of that when the
  // block partials need more (equal rounds; the output head fits in one)
  nwg = Q6D_TARGET_WGS;
  const int64_t need = (units + cap_units - 1) / cap_units;
  if (need > nwg) nwg = (need + Q6D_TARGET_WGS - 1) / Q6D_TARGET_WGS * Q6D_TARGET_WGS;
  if (nwg > units) nwg = units;
  units_q = (int)(units / nwg);
  units_rem = (int)(units % nwg);
  const int64_t max_blocks = (int64_t)(units_q + (units_rem ? 1 : 0)) * unit * nb;
  lds = fixed + (size_t)max_blocks * 4;
  return lds <= Q6D_LDS_LIMIT && max_blocks < 65536 && K / 8 <= 32 * Q6D_THREADS;
}

template <int XC>
void q6_launch_dense(const void *w, const void *x, float *y, int64_t N, int64_t K, int unit,
                     int units_q, int units_rem, int64_t nwg, size_t lds, hipStream_t s) {
  auto kern = q6k_gemv_m1_kernel<XC>;
  (void)hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
  const uint32_t nb = (uint32_t)(K / QK);
  const uint32_t magic = nb > 1 ? (uint32_t)((((uint64_t)1 << 32) + nb - 1) / nb) : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(Q6D_THREADS), lds, s, (const uint8_t *)w,
                     (const uint16_t *)x, y, (int)K, unit, units_q, units_rem, (int)N, magic);
}

// The dense kernel for M = 1 with bf16 x, or false if its plan does not fit.
bool q6_try_dense(const void *w, const void *x, float *y, int64_t N, int64_t K, hipStream_t s) {
  int unit, units_q, units_rem;
  int64_t nwg;
  size_t lds;
  if (!q6_dense_plan(N, K, unit, units_q, units_rem, nwg, lds)) return false;
  const int64_t xc = (K / 8 + Q6D_THREADS - 1) / Q6D_THREADS;
  if (xc <= 2)
    q6_launch_dense<2>(w, x, y, N, K, unit, units_q, units_rem, nwg, lds, s);
  else if (xc <= 4)
    q6_launch_dense<4>(w, x, y, N, K, unit, units_q, units_rem, nwg, lds, s);
  else if (xc <= 8)
    q6_launch_dense<8>(w, x, y, N, K, unit, units_q, units_rem, nwg, lds, s);
  else if (xc <= 16)
    q6_launch_dense<16>(w, x, y, N, K, unit, units_q, units_rem, nwg, lds, s);
  else
    q6_launch_dense<32>(w, x, y, N, K, unit, units_q, units_rem, nwg, lds, s);
  return true;
}

}  // namespace

void launch_q80_mfma_gemv(const void *w, const uint16_t *x, float *y, int64_t M, int64_t N,
                          int64_t K, hipStream_t s) {
  launch_kq_mfma<MfQ8>(w, x, y, M, N, K, s);
}

void launch_q4k_mfma_gemv(const void *w, const uint16_t *x, float *y, int64_t M, int64_t N,
                          int64_t K, bool q5, hipStream_t s) {
  if (q5)
    launch_kq_mfma<MfQ4<true>>(w, x, y, M, N, K, s);
  else
    launch_kq_mfma<MfQ4<false>>(w, x, y, M, N, K, s);
}

void launch_q6k_gemv(const void *w, const void *x, bool x_bf16, float *y, int64_t M,
                     int64_t N, int64_t K, hipStream_t s) {
  // M = 1, bf16 x: the dense-span kernel whenever its plan fits (K up to about
  // 30K). It runs the down shape K = 17408, N = 5120 in about 16 us and the
  // output head K = 5120, N = 151936 in about 97-104 us, against 25.5 us and
  // 136-138 us for the VALU kernel's forms (which hand out whole row groups).
  if (M == 1 && x_bf16 && ((uintptr_t)w & 15) == 0 && q6_try_dense(w, x, y, N, K, s)) return;
  if (x_bf16 && M >= Q6_MFMA_MIN_M) {
    launch_kq_mfma<MfQ6>(w, (const uint16_t *)x, y, M, N, K, s);
    return;
  }
  const size_t per_row = (size_t)K * (x_bf16 ? 2 : 4) + (size_t)(K / 16) * 4;
  const size_t elt = x_bf16 ? 2 : 4;
  int64_t m0 = 0;
  while (m0 < M) {
    const int64_t rem = M - m0;
    int mt = 8;
    while (mt > 1 && (mt > rem || (size_t)mt * per_row > 150 * 1024)) mt >>= 1;
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
