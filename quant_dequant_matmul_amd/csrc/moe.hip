// Routed MoE FFN with Q4_K experts, one call per layer (expert-grouped
// matmul; hipster README, "Verify the claims": MoE grouped GEMM). The down
// experts may also be Q5_K, the expert-down type of a Q4_K_M file (hipEngine
// README, "GGUF Support", payload table).
//
//   y_t = sum_s gw[t][s] * W2[e] * (silu(W13[e][0:F] x_t) * W13[e][F:2F] x_t),
//   e = ids[t][s]   (entries whose id is outside [0, E) contribute nothing).
//
// Two regimes, chosen on the host from the entry count n = T * top_k.
//
// Decode (n <= 64): every workgroup routes the few entries itself (bitmap of
// the experts present; the a-th of them in increasing id order; its entries
// in (t, s) order), so there is no routing launch. Workgroup (chunk, a)
// streams its row chunk of the a-th active expert's weights once and
// multiplies it with all that expert's entries, whose inputs it holds in LDS.
//  1. gate+up+SwiGLU: rows f of the gate half and F + f of the up half in one
//     workgroup; h[entry][f] = silu(g) * u, fp32.
//  2. down: o[entry][r], fp32.
//  3. combine: y[t][r] = sum over s in slot order of gw[t][s] * o[t*k+s][r].
//
// Matrix cores (n > 64):
//  1. route (one workgroup): histogram of the ids, exclusive scan, stable
//     scatter of the entries into expert order (perm).
//  2. gate+up+SwiGLU: workgroup (f tile of 128, e) decodes 128 gate rows and
//     the matching 128 up rows of W13[e] to bf16 in LDS, 64 K at a time, and
//     multiplies them with up to 128 gathered x rows of e's entries per pass
//     (v_mfma_f32_32x32x16_bf16, fp32 accumulators); the gate and up values
//     of one (entry, f) land in the same lane, so h = silu(g) * u is formed
//     in registers and stored as bf16 by entry.
//  3. down: workgroup (row tile of 256, e): W2[e] rows times the h rows of
//     e's entries -> o[entry][r], fp32.
//  4. combine as above.
#include <mutex>

#include "common.h"
#include "launch.h"
#include "q4k_tile.h"

#include <type_traits>

// Scratch of the no-allocation MoE entry point: the workspace of one call
// lives in this device array (every GPU the library runs on holds its own copy
// until the process ends). Host code never uses the array's name as an
// address: it takes each device's copy through hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[qdm::MOE_SCRATCH_BYTES];

namespace qdm {

namespace {


inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// Decode regime (n = T * top_k <= 64 entries).
// ---------------------------------------------------------------------------
constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / WAVE;
constexpr int DEC_MAX_N = 64;
constexpr int DEC_PF = 3;  // wave iterations of weight loads in flight
// Rows per decode workgroup: gate/up row pairs (FR) and W2 rows (RW). Few
// tokens touch few experts, and small workgroups spread them over more compute
// units; from 4 tokens on, larger workgroups spend less on their fixed costs
// (measured at H = 2048, F = 768, 128 experts, top-8).
constexpr int DEC_FR_SMALL = 16, DEC_RW_SMALL = 64;
// A single token: 8 row pairs per gate+up workgroup (twice the workgroups;
// 17.0 -> 16.4 us at T = 1, but 21.8 -> 24.3 us at T = 2)
constexpr int DEC_FR_ONE = 8;
constexpr int DEC_FR_LARGE = 32, DEC_RW_LARGE = 128;
constexpr int DEC_LARGE_FROM_T = 4;
constexpr int DEC_MT_MAX = 4;  // entries per pass (more entries of one expert take more passes)

// A value the compiler cannot see through (keeps v_and_or_b32 forms).
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Routing of at most 64 entries, derived by every workgroup from the ids:
// the number of distinct valid experts, the a-th of them in increasing id
// order (-1 past the end), its entries in increasing (t, s) order, and the
// number of entries whose id is outside [0, E).
struct SmallRoute {
  int nact, e, cnt, bad;
  int ent[DEC_MAX_N];
};

__device__ void small_route(const int32_t *__restrict__ ids, int n, int E, int a, SmallRoute &sr,
                            uint32_t *bitmap) {
  const int tid = threadIdx.x;
  if (tid < 32) bitmap[tid] = 0u;  // E <= 1024 experts: 32 words
  __syncthreads();
  int myid = -1;
  if (tid < WAVE) {
    if (tid < n) myid = ids[tid];
    if (myid >= 0 && myid < E) atomicOr(&bitmap[myid >> 5], 1u << (myid & 31));
  }
  __syncthreads();
  if (tid < WAVE) {
    const uint32_t word = tid < 32 ? bitmap[tid] : 0u;
    const int c = __popc(word);
    int incl = c;  // inclusive prefix of set bits over words
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const int v = __shfl_up(incl, o, WAVE);
      if (tid >= o) incl += v;
    }
    const int total = __shfl(incl, 31, WAVE);
    const int excl = incl - c;
    const uint64_t hm = __ballot(tid < 32 && a >= excl && a < incl);
    int e = -1;
    if (hm != 0ull) {
      const int L = __builtin_ctzll(hm);
      uint32_t wl = (uint32_t)__shfl((int)word, L, WAVE);
      const int r = a - __shfl(excl, L, WAVE);
      for (int i = 0; i < r; i++) wl &= wl - 1u;  // drop the r lowest set bits
      e = 32 * L + __builtin_ctz(wl);
    }
    const bool mine = e >= 0 && tid < n && myid == e;
    const uint64_t mm = __ballot(mine);
    const uint64_t bad = __ballot(tid < n && (myid < 0 || myid >= E));
    if (mine) sr.ent[__popcll(mm & ((1ull << tid) - 1ull))] = tid;
    if (tid == 0) {
      sr.nact = total;
      sr.e = e;
      sr.cnt = __popcll(mm);
      sr.bad = __popcll(bad);
    }
  }
  __syncthreads();
}

// Stages mt input rows of length K into LDS: bf16 rows as (x0, x2, x1, x3)
// groups (to match the code pairs of the dot below) or fp32 rows as they are,
// plus every row's 32-element sums. Row m is src_row(m). Every 64-element
// piece (what one lane reads for its code chunk) is padded by 16 bytes, so
// the 16 (column block, chunk) pieces a wave reads at once start on 16
// different LDS bank groups.
constexpr int PIECE_BF16 = 128 + 16, REC_BF16 = 4 * PIECE_BF16;  // bytes per 64 / 256 bf16
constexpr int PIECE_F32 = 256 + 16, REC_F32 = 4 * PIECE_F32;     // bytes per 64 / 256 fp32

template <bool XBF16, typename SrcRow>
__device__ __forceinline__ void stage_rows(SrcRow src_row, int mt, int K, uint8_t *lds_in,
                                           float *lds_sum) {
  constexpr int PER_CHUNK = XBF16 ? 8 : 4;   // elements per 16-byte chunk
  constexpr int CH_PER_SUM = 32 / PER_CHUNK;
  constexpr int CH_PER_PIECE = 64 / PER_CHUNK;
  constexpr int PIECE = XBF16 ? PIECE_BF16 : PIECE_F32;
  const int rchunks = K / PER_CHUNK;
  const int nchunk = mt * rchunks;
  const int rowb = (K / 64) * PIECE;
  for (int base = 0; base < nchunk; base += DEC_THREADS) {
    const int cidx = base + threadIdx.x;
    float s = 0.f;
    if (cidx < nchunk) {
      const int m = cidx / rchunks, cc = cidx - m * rchunks;
      const u32x4 v = ((const u32x4 *)src_row(m))[cc];
      uint8_t *dst = lds_in + m * rowb + (cc / CH_PER_PIECE) * PIECE + (cc % CH_PER_PIECE) * 16;
      if constexpr (XBF16) {
        u32x4 p;
        p.x = (v.x & 0xFFFFu) | (v.y << 16);
        p.y = (v.x >> 16) | (v.y & 0xFFFF0000u);
        p.z = (v.z & 0xFFFFu) | (v.w << 16);
        p.w = (v.z >> 16) | (v.w & 0xFFFF0000u);
        *(u32x4 *)dst = p;
        s = bf16_bits_to_float(v.x) + bf16_bits_to_float(v.x >> 16) +
            bf16_bits_to_float(v.y) + bf16_bits_to_float(v.y >> 16) +
            bf16_bits_to_float(v.z) + bf16_bits_to_float(v.z >> 16) +
            bf16_bits_to_float(v.w) + bf16_bits_to_float(v.w >> 16);
      } else {
        *(u32x4 *)dst = v;
        const f32x4 f = __builtin_bit_cast(f32x4, v);
        s = (f.x + f.y) + (f.z + f.w);
      }
    }
    s = lane_group_sum<CH_PER_SUM>(s);
    if (cidx < nchunk && (cidx % CH_PER_SUM) == 0) lds_sum[cidx / CH_PER_SUM] = s;
  }
}

// part[m][b] = sum over block b's 256 weights of w * in_m, for the nblk blocks
// blk_ptr(0 .. nblk-1) (block b covers input columns (b % nb) * 256 ..) and
// the mt staged rows. 4 lanes per block (lane c owns code chunk c, sub-blocks
// 2c and 2c+1), 16 blocks per wave iteration, DEC_PF iterations of loads in
// flight; loads are unconditional (clamped) so waits are exact. prefetch()
// issues the first loads (before the inputs are staged), run() the rest.
// Q5 = true reads Q5_K blocks (176 B: the Q4_K header, a 32-byte high-bit
// plane at 16, the code bytes at 48); each lane then also loads the plane and
// merges bits 2c and 2c+1 into its code bytes.
template <bool XBF16, int MT, bool Q5, typename BlkPtr>
struct RowsDot {
  static constexpr int QOFF = Q5 ? 48 : 16;
  BlkPtr blk_ptr;
  int nblk, wb0, wb1, iters, g, c;
  u32x4 Hd[DEC_PF], A[DEC_PF], Bq[DEC_PF];
  u32x4 Ha[Q5 ? DEC_PF : 1], Hb[Q5 ? DEC_PF : 1];

  __device__ __forceinline__ RowsDot(BlkPtr bp, int nblk_) : blk_ptr(bp), nblk(nblk_) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    g = lane >> 2;
    c = lane & 3;
    wb0 = wave * nblk / DEC_WAVES;
    wb1 = (wave + 1) * nblk / DEC_WAVES;
    iters = (wb1 - wb0 + 15) >> 4;
  }

  __device__ __forceinline__ void load(int slot, int it) {
    const uint8_t *blk = blk_ptr(min(wb0 + g + 16 * it, wb1 - 1));
    Hd[slot] = *(const u32x4 *)blk;
    A[slot] = *(const u32x4 *)(blk + QOFF + 32 * c);
    Bq[slot] = *(const u32x4 *)(blk + QOFF + 16 + 32 * c);
    if constexpr (Q5) {
      Ha[slot] = *(const u32x4 *)(blk + 16);
      Hb[slot] = *(const u32x4 *)(blk + 32);
    }
  }

  __device__ __forceinline__ void prefetch() {
    if (iters == 0) return;
#pragma unroll
    for (int p = 0; p < DEC_PF; p++) load(p, min(p, iters - 1));
  }

  __device__ __forceinline__ void run(int nb, int K, int mt, const uint8_t *lds_in,
                                      const float *lds_sum, float *part) {
    constexpr int REC = XBF16 ? REC_BF16 : REC_F32;
    constexpr int PIECE = XBF16 ? PIECE_BF16 : PIECE_F32;
    if (iters == 0) return;
    // Q4_K codes are nibbles picked straight from the code words; Q5_K codes
    // are assembled into bytes (nibble | high bit << 4) first
    const uint32_t MASK = opaque_u32(Q5 ? 0x00FF00FFu : 0x000F000Fu);
    const uint32_t MAGIC = opaque_u32(0x43004300u);
    // column block of the lane's block, stepped by 16 blocks per iteration
    const int s16 = 16 % nb;
    int kb = (wb0 + g) % nb;
    for (int it0 = 0; it0 < iters; it0 += DEC_PF) {
#pragma unroll
      for (int p = 0; p < DEC_PF; p++) {
        const int it = it0 + p;
        if (it < iters) {
          const int b = wb0 + g + 16 * it;
          const bool valid = b < wb1;
          const u32x4 hdr = Hd[p];
          const uint32_t q[8] = {A[p].x, A[p].y, A[p].z, A[p].w,
                                 Bq[p].x, Bq[p].y, Bq[p].z, Bq[p].w};
          // code words of sub-blocks 2c (lo) and 2c+1 (hi), positions 4i .. 4i+3
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
          load(p, min(it + DEC_PF, iters - 1));  // refill the slot right away
          const float d = half_bits_to_float(hdr.x), dmin = half_bits_to_float(hdr.x >> 16);
          uint32_t sc0, m0, sc1, m1;
          q4k_scale_min(hdr.y, hdr.z, hdr.w, 2 * c, sc0, m0);
          q4k_scale_min(hdr.y, hdr.z, hdr.w, 2 * c + 1, sc1, m1);
          const float a0 = d * (float)sc0, b0 = dmin * (float)m0;
          const float a1 = d * (float)sc1, b1 = dmin * (float)m1;
          const int e0 = kb * QK + 64 * c;  // first input column of sub-block 2c
#pragma unroll
          for (int m = 0; m < MT; m++) {
            if (m < mt) {
              const float2 xs = *(const float2 *)(lds_sum + m * (K / 32) + (e0 >> 5));
              float s0 = 0.f, s1 = 0.f, r;
              if constexpr (XBF16) {
                const u32x4 *xv = (const u32x4 *)(lds_in + (m * nb + kb) * REC + PIECE * c);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                  const u32x4 x0 = xv[i], x1 = xv[4 + i];
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
                r = a0 * s0;
                r = fmaf(-fmaf(128.f, a0, b0), xs.x, r);
                r = fmaf(a1, s1, r);
                r = fmaf(-fmaf(128.f, a1, b1), xs.y, r);
              } else {
                const f32x4 *xv = (const f32x4 *)(lds_in + (m * nb + kb) * REC + PIECE * c);
#pragma unroll
                for (int i = 0; i < 8; i++) {
                  const f32x4 x0 = xv[i], x1 = xv[8 + i];
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
                r = a0 * s0;
                r = fmaf(-b0, xs.x, r);
                r = fmaf(a1, s1, r);
                r = fmaf(-b1, xs.y, r);
              }
              r = lane_group_sum<4>(r);
              if (valid && c == 0) part[m * nblk + b] = r;
            }
          }
          kb += s16;
          if (kb >= nb) kb -= nb;
        }
      }
    }
  }
};

template <bool XBF16, int MT, bool Q5, typename BlkPtr>
__device__ __forceinline__ RowsDot<XBF16, MT, Q5, BlkPtr> make_rows_dot(BlkPtr bp, int nblk) {
  return RowsDot<XBF16, MT, Q5, BlkPtr>(bp, nblk);
}

// ---------------------------------------------------------------------------
// Router: top-k experts and their softmax gate weights from router logits.
// ---------------------------------------------------------------------------
// One wave per token; lane l holds logits l, l+64, ... (E <= 64 * PER). Each
// logit becomes a 64-bit key: the logit's bits mapped to an unsigned integer
// of the same order (-0 taken as +0, so equal logits give equal high words),
// and ~e in the low word, so that the largest key is the largest logit and,
// among equal logits, the smallest index. Each of the k rounds takes the
// wave's largest key (lane-local maximum, DPP maxima within each row of 16
// lanes, then the four row results read out), and the lane holding it clears
// that key. Lane s keeps winner s; the gate weights are the softmax of the k
// winners, exp(l_s - l_0) / sum_j exp(l_j - l_0) with l_0 the largest (no
// overflow for large logits).
constexpr int RT_THREADS = 256;
constexpr int RT_MAX_E = 1024, RT_MAX_K = 16;
static_assert(RT_MAX_K <= 16, "the winners are gathered in the 16 lanes of row 0");

// DPP controls (row = 16 lanes): swap neighbours, swap pairs, mirror within
// each half row, mirror within the row.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t a) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)a, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(a >> 32), CTRL, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
  return o > a ? o : a;
}

template <int CTRL>
__device__ __forceinline__ float dpp_add_f32(float a) {
  return a + __int_as_float(
                 __builtin_amdgcn_update_dpp(0, __float_as_int(a), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ uint64_t rd_lane_u64(uint64_t a, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)a, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(a >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float order_bits_inv(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// The router for one token, by one whole wave: logits lt[0 .. E-1]
// (E <= 64 * PER) -> ids[s], gw[s] for s < k, written by lane s.
template <int PER>
__device__ __forceinline__ void router_one(const float *__restrict__ lt, int E, int k, int lane,
                                           int32_t *ids, float *gw) {
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; j++) v[j] = lt[min(lane + WAVE * j, E - 1)];  // all loads in flight
  uint64_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; j++) {
    const int e = lane + WAVE * j;
    key[j] = e < E ? ((uint64_t)order_bits(v[j]) << 32) | (uint32_t)~(uint32_t)e : 0;
  }
  uint64_t mine = 0;  // lane s: the key of winner s
  for (int s = 0; s < k; s++) {
    uint64_t m = key[0];
#pragma unroll
    for (int j = 1; j < PER; j++) m = key[j] > m ? key[j] : m;
    m = dpp_max_u64<DPP_XOR1>(m);
    m = dpp_max_u64<DPP_XOR2>(m);
    m = dpp_max_u64<DPP_HALF_MIRROR>(m);
    m = dpp_max_u64<DPP_MIRROR>(m);
    uint64_t best = rd_lane_u64(m, 0);
#pragma unroll
    for (int r = 1; r < 4; r++) {
      const uint64_t o = rd_lane_u64(m, 16 * r);
      best = o > best ? o : best;
    }
#pragma unroll
    for (int j = 0; j < PER; j++)
      if (key[j] == best) key[j] = 0;  // the winner's key exists once (the index is in it)
    if (lane == s) mine = best;
  }
  // k <= 16: the winners sit in lanes 0..k-1 of row 0.
  const float l0 = order_bits_inv((uint32_t)(rd_lane_u64(mine, 0) >> 32));
  float ex = lane < k ? expf(order_bits_inv((uint32_t)(mine >> 32)) - l0) : 0.f;
  float sum = dpp_add_f32<DPP_XOR1>(ex);
  sum = dpp_add_f32<DPP_XOR2>(sum);
  sum = dpp_add_f32<DPP_HALF_MIRROR>(sum);
  sum = dpp_add_f32<DPP_MIRROR>(sum);
  if (lane < k) {
    ids[lane] = (int32_t)~(uint32_t)mine;
    gw[lane] = ex / sum;
  }
}

// Decode gate+up+SwiGLU: workgroup (f chunk, a) with e = the a-th active
// expert; rows f0 .. f0+fr-1 (gate) and F+f0 .. (up) of W13[e], all entries
// of e; h[entry][f] = silu(g) * u (fp32).
// LG (router logits [T][E], E <= 128): every workgroup first runs the router
// itself, one wave per token, into LDS, and routes from there; workgroup
// (0, 0) also writes the ids and gate weights to ids_out / gw_out for the
// down and combine kernels (the router fused into this kernel).
template <int MT, int DEC_FR, bool LG>
__global__ __launch_bounds__(DEC_THREADS) void moe_dec_gateup_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w13,
    const int32_t *__restrict__ ids, int n, int top_k, int E, int H, int F,
    float *__restrict__ h, const float *__restrict__ logits, int32_t *__restrict__ ids_out,
    float *__restrict__ gw_out, uint32_t *__restrict__ status) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ SmallRoute sr;
  __shared__ uint32_t bitmap[32];
  __shared__ int32_t lg_ids[LG ? DEC_MAX_N : 1];
  __shared__ float lg_gw[LG ? DEC_MAX_N : 1];
  const int32_t *rid = ids;
  if constexpr (LG) {
    const int T = n / top_k, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int t = wv; t < T; t += DEC_THREADS / WAVE)  // uniform per wave
      router_one<2>(logits + (int64_t)t * E, E, top_k, lane, lg_ids + t * top_k,
                    lg_gw + t * top_k);
    __syncthreads();
    if (blockIdx.x == 0 && blockIdx.y == 0 && (int)threadIdx.x < n) {
      ids_out[threadIdx.x] = lg_ids[threadIdx.x];
      gw_out[threadIdx.x] = lg_gw[threadIdx.x];
    }
    rid = lg_ids;
  }
  small_route(rid, n, E, blockIdx.y, sr, bitmap);
  // the call's count of skipped ids (every workgroup derives the same value)
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) status[0] = (uint32_t)sr.bad;
  if (sr.e < 0) return;
  const int e = sr.e, cnt = sr.cnt;
  const int nb = H / QK;
  const int f0 = blockIdx.x * DEC_FR, fr = min(DEC_FR, F - f0);
  const int nrows = 2 * fr, nblk = nrows * nb;
  uint8_t *lds_in = (uint8_t *)lds;                       // [MT][nb][REC_BF16]
  float *lds_sum = (float *)(lds_in + MT * nb * REC_BF16);  // [MT][H / 32]
  float *part = lds_sum + MT * (H / 32);                  // [MT][2 DEC_FR nb]
  float *res = part + MT * 2 * DEC_FR * nb;               // [MT][2 DEC_FR]
  const uint8_t *we = w13 + (int64_t)e * 2 * F * nb * Q4K_BYTES;
  auto blk_ptr = [&](int b) {  // gate rows first, then the matching up rows
    const int r = b / nb;
    const int row = r < fr ? f0 + r : F + f0 + (r - fr);
    return we + ((int64_t)row * nb + (b - r * nb)) * Q4K_BYTES;
  };
  auto rd = make_rows_dot<true, MT, false>(blk_ptr, nblk);
  for (int c0 = 0; c0 < cnt; c0 += MT) {
    const int mt = min(MT, cnt - c0);
    rd.prefetch();  // weight loads fly while the x rows are staged
    stage_rows<true>([&](int m) { return x + (int64_t)(sr.ent[c0 + m] / top_k) * H; }, mt, H,
                     lds_in, lds_sum);
    __syncthreads();
    rd.run(nb, H, mt, lds_in, lds_sum, part);
    __syncthreads();
    for (int t = threadIdx.x; t < mt * nrows; t += DEC_THREADS) {  // rows in block order
      const int m = t / nrows, r = t - m * nrows;
      const float *pp = part + m * nblk + r * nb;
      float sacc = 0.f;
      for (int k = 0; k < nb; k++) sacc += pp[k];
      res[m * nrows + r] = sacc;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < mt * fr; t += DEC_THREADS) {
      const int m = t / fr, f = t - m * fr;
      const float gt = res[m * nrows + f], up = res[m * nrows + fr + f];
      h[(int64_t)sr.ent[c0 + m] * F + f0 + f] = gt / (1.0f + expf(-gt)) * up;
    }
    __syncthreads();
  }
}

// Decode down: workgroup (row chunk, a): o[entry][r] for rows r0 .. r0+rw-1
// of W2[e] and every entry of e (fp32). W2 is Q4_K, or Q5_K when Q5.
template <int MT, int DEC_RW, bool Q5>
__global__ __launch_bounds__(DEC_THREADS) void moe_dec_down_kernel(
    const float *__restrict__ h, const uint8_t *__restrict__ w2, const int32_t *__restrict__ ids,
    float *__restrict__ o, int n, int top_k, int E, int H, int F) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ SmallRoute sr;
  __shared__ uint32_t bitmap[32];
  small_route(ids, n, E, blockIdx.y, sr, bitmap);
  const int r0 = blockIdx.x * DEC_RW, rw = min(DEC_RW, H - r0);
  if (sr.e < 0) return;
  const int e = sr.e, cnt = sr.cnt;
  const int nb = F / QK, nblk = rw * nb;
  uint8_t *lds_in = (uint8_t *)lds;                       // [MT][nb][REC_F32]
  float *lds_sum = (float *)(lds_in + MT * nb * REC_F32);  // [MT][F / 32]
  float *part = lds_sum + MT * (F / 32);           // [MT][DEC_RW nb]
  constexpr int BB = Q5 ? Q5K_BYTES : Q4K_BYTES;
  const uint8_t *rows = w2 + ((int64_t)e * H + r0) * nb * BB;
  auto blk_ptr = [&](int b) { return rows + (int64_t)b * BB; };
  auto rd = make_rows_dot<false, MT, Q5>(blk_ptr, nblk);
  for (int c0 = 0; c0 < cnt; c0 += MT) {
    const int mt = min(MT, cnt - c0);
    rd.prefetch();  // weight loads fly while the h rows are staged
    stage_rows<false>([&](int m) { return h + (int64_t)sr.ent[c0 + m] * F; }, mt, F, lds_in,
                      lds_sum);
    __syncthreads();
    rd.run(nb, F, mt, lds_in, lds_sum, part);
    __syncthreads();
    for (int t = threadIdx.x; t < mt * rw; t += DEC_THREADS) {
      const int m = t / rw, r = t - m * rw;
      const float *pp = part + m * nblk + r * nb;
      float sacc = 0.f;
      for (int k = 0; k < nb; k++) sacc += pp[k];
      o[(int64_t)sr.ent[c0 + m] * H + r0 + r] = sacc;
    }
    __syncthreads();
  }
}

// y[t][r] = sum over slots s in order of gw[t][s] * o[t*top_k+s][r], slots
// with an id outside [0, E) skipped (o is indexed by entry). The loads of a
// group of up to 8 slots (id, gate weight, 4 outputs) are all issued before
// any is used: their addresses do not depend on the ids (every entry's o row
// exists), so a call waits about one memory latency per group instead of
// several in a row; an invalid slot is masked afterwards (its o row may hold
// anything: it is never multiplied).
__global__ __launch_bounds__(256) void moe_combine_entries_kernel(
    const float *__restrict__ o, const int32_t *__restrict__ ids, const float *__restrict__ gw,
    float *__restrict__ y, int T, int top_k, int E, int H) {
  // one thread per token t and 4 consecutive outputs (H % 4 == 0)
  constexpr int G = 8;
  const int h4 = H / 4;
  const int64_t total = (int64_t)T * h4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / h4;
    const int c = (int)(i - t * h4);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < top_k; s0 += G) {
      int id[G];
      float g[G];
      f32x4 v[G];
#pragma unroll
      for (int j = 0; j < G; j++) {
        const int64_t en = t * top_k + min(s0 + j, top_k - 1);
        id[j] = ids[en];
        g[j] = gw[en];
        v[j] = *(const f32x4 *)(o + en * H + 4 * c);
      }
#pragma unroll
      for (int j = 0; j < G; j++) {
        if (s0 + j < top_k && id[j] >= 0 && id[j] < E) {
          acc.x = fmaf(g[j], v[j].x, acc.x);
          acc.y = fmaf(g[j], v[j].y, acc.y);
          acc.z = fmaf(g[j], v[j].z, acc.z);
          acc.w = fmaf(g[j], v[j].w, acc.w);
        }
      }
    }
    *(f32x4 *)(y + t * H + 4 * c) = acc;
  }
}

template <int PER>
__global__ __launch_bounds__(RT_THREADS) void moe_router_topk_kernel(
    const float *__restrict__ logits, int T, int E, int k, int32_t *__restrict__ ids,
    float *__restrict__ gw) {
  const int lane = threadIdx.x & 63;
  const int t = (int)blockIdx.x * (RT_THREADS / WAVE) + (int)(threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave: the DPP steps see all 64 lanes
  router_one<PER>(logits + (int64_t)t * E, E, k, lane, ids + (int64_t)t * k, gw + (int64_t)t * k);
}

// ---------------------------------------------------------------------------
// Matrix-core regime (n > 64).
// ---------------------------------------------------------------------------
constexpr int ROUTE_THREADS = 1024;
constexpr int ROUTE_WAVES = ROUTE_THREADS / WAVE;
constexpr int ROUTE_IDS = 4;  // ids per thread and batch

// One workgroup: offsets[e] = first sorted position of expert e (exclusive
// scan of the counts, offsets[E] = valid entries), perm[pos] = entry index
// for the entries of e at positions offsets[e] .. offsets[e+1]-1. Within an
// expert the order is whatever order the LDS atomics hand out positions in:
// an entry's outputs do not depend on where it sits among its expert's
// entries (each output row of the matrix-core kernels is its own dot
// product, and the combine sums an entry's slots in slot order), so the
// results are the same bit for bit whatever that order.
__global__ __launch_bounds__(ROUTE_THREADS) void moe_route_kernel(
    const int32_t *__restrict__ ids, int n, int E, int32_t *__restrict__ offsets,
    int32_t *__restrict__ perm, uint32_t *__restrict__ status) {
  extern __shared__ int32_t rsm[];
  int32_t *run = rsm;  // [E] counts, then running positions
  __shared__ int32_t wsum[ROUTE_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // ids are read once per batch of ROUTE_IDS chunks (all loads in flight
  // together) and serve both the histogram and the scatter
  int idr[ROUTE_IDS];
  auto load_batch = [&](int base) {
#pragma unroll
    for (int j = 0; j < ROUTE_IDS; j++) {
      const int i = base + ROUTE_THREADS * j + tid;
      const int id = i < n ? ids[i] : -1;
      idr[j] = (id >= 0 && id < E) ? id : -1;
    }
  };
  for (int e = tid; e < E; e += ROUTE_THREADS) run[e] = 0;
  __syncthreads();
  constexpr int BATCH = ROUTE_THREADS * ROUTE_IDS;
  for (int base = 0; base < n; base += BATCH) {
    load_batch(base);
#pragma unroll
    for (int j = 0; j < ROUTE_IDS; j++)
      if (idr[j] >= 0) atomicAdd(&run[idr[j]], 1);
  }
  __syncthreads();
  const int v = tid < E ? run[tid] : 0;  // E <= 1024: one count per thread
  int incl = v;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const int u = __shfl_up(incl, o, WAVE);
    if (lane >= o) incl += u;
  }
  if (lane == WAVE - 1) wsum[wave] = incl;
  __syncthreads();
  int wpre = 0, total = 0;
  for (int w = 0; w < ROUTE_WAVES; w++) {
    if (w < wave) wpre += wsum[w];
    total += wsum[w];
  }
  if (tid < E) {
    offsets[tid] = wpre + incl - v;
    run[tid] = wpre + incl - v;
  }
  if (tid == 0) {
    offsets[E] = total;
    status[0] = (uint32_t)(n - total);  // entries skipped: id outside [0, E)
  }
  __syncthreads();
  for (int base = 0; base < n; base += BATCH) {
    if (n > BATCH) load_batch(base);  // a single batch is still in registers
#pragma unroll
    for (int j = 0; j < ROUTE_IDS; j++) {
      const int i = base + ROUTE_THREADS * j + tid;
      if (idr[j] >= 0) perm[atomicAdd(&run[idr[j]], 1)] = i;
    }
  }
}

constexpr int MX_THREADS = 512;  // eight waves: one workgroup per compute unit
constexpr int MX_WROWS = 64;     // weight rows per wave pair: two 32-row MFMA tiles
constexpr int MX_PASS = 64;      // entries per pass: one or two 32-row MFMA tiles
constexpr int MX_ASLOTS = 33;    // 16-byte LDS slots per A row: a block's 32, one of padding
constexpr int MX_ABYTES = MX_PASS * MX_ASLOTS * 16;  // one A buffer: 33,792 B
constexpr int mx_wbytes(bool q5) { return 4 * MX_WROWS * (q5 ? Q5K_BYTES : Q4K_BYTES); }

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// One pass over up to MX_PASS entries (MS tiles of 32) of the workgroup's
// 256 weight rows. Waves w and w+4 (one SIMD) own the same 64 rows: wave w
// multiplies chunks 0 and 1 of every block, wave w+4 chunks 2 and 3, and at
// the end of the pass wave w+4 hands its sums to wave w through LDS. Block by
// block: at the top of block b every wave waits for its copies of block b, a
// barrier makes all of them visible, the copies of block b+1 into the other
// buffers are issued, and block b is multiplied.
// Copies go from global memory straight into LDS (global_load_lds_dwordx4), a
// wave's 64 lanes writing 1 KiB of consecutive LDS:
//   weights: row group g's rows (64 per group), block b of each (BB bytes,
//     BB/16 pieces), piece p = 64i + lane of copy i at LDS byte 16p of the
//     group's area (row-major, BB per row); the group's two waves take the
//     even and the odd copies;
//   A: entry row r of the pass, its 256 k of block b (512 bytes) in slots
//     33r .. 33r+31 (slot 33r+32 is padding: rows 528 bytes apart keep the
//     16-byte reads below free of bank conflicts), slot s = 64(8i + wave) +
//     lane of copy i. Rows past the pass's entries repeat its last entry.
// Lane (n, h) = (lane % 32, lane / 32) reads its rows' code bytes and its A
// pieces from LDS and multiplies as follows. The reduction order over K is
// free, so K is permuted to suit the code layout: in chunk c of a block
// (sub-blocks 2c and 2c+1), code byte l holds weight 64c + l in its low nibble
// and 64c + 32 + l in its high nibble; lane half h takes bytes 16h .. 16h+15,
// and the four MFMA steps of the chunk take, from those bytes, the low
// nibbles of bytes 0..7, of 8..15, then the high nibbles of 0..7, of 8..15.
// The A operand of step t then holds x at k = 64c + 32(t/2) + 16h + 8(t%2)
// .. +7: one 16-byte LDS read. The weights are decoded in registers straight
// into the B operand; nothing decoded goes through LDS.
template <bool GATEUP, bool Q5, int MS>
__device__ __forceinline__ void mx_pass(const uint16_t *__restrict__ a_src,
                                        const uint8_t *const (&wsrc)[(Q5 ? 11 : 9) / 2 + 1],
                                        const int32_t *__restrict__ pent, int rows, int top_k,
                                        int K, int ldo, int col0, uint16_t *__restrict__ hb,
                                        float *__restrict__ o, uint8_t *const (&sw)[2],
                                        uint8_t *const (&sa)[2]) {
  constexpr int BB = Q5 ? Q5K_BYTES : Q4K_BYTES;
  constexpr int NP = BB / 16;         // 16-byte pieces per block
  constexpr int QOFF = Q5 ? 48 : 16;  // first code byte of a block
  constexpr int NA = (MS * 32 * MX_ASLOTS + 63) / 64;  // A copies per block (all waves)
  constexpr int NAW = (NA + 7) / 8;                    // A copies per wave, at most
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const int grp = wave & 3, kh = wave >> 2;
  const int nbk = K / QK;
  // A copy sources: slot s of copy i is piece s % 33 (the padding slot copies
  // piece 31 again) of entry row s / 33
  const uint16_t *asrc[NAW];
#pragma unroll
  for (int i = 0; i < NAW; i++) {
    const int s = 64 * (8 * i + wave) + lane;
    const int r = min(s / MX_ASLOTS, rows - 1);
    const int ent = pent[r];
    asrc[i] = a_src + (int64_t)(GATEUP ? ent / top_k : ent) * K + 8 * min(s % MX_ASLOTS, 31);
  }
  // A first: its sources depend on the entry loads, and waiting for those
  // then waits for no weight copy
  auto copy_block = [&](int b, uint8_t *w, uint8_t *a) {
#pragma unroll
    for (int i = 0; i < NAW; i++)
      if (8 * i + wave < NA)  // uniform
        __builtin_amdgcn_global_load_lds((const void *)(asrc[i] + QK * b),
                                         (lds_ptr_t)(a + 1024 * (8 * i + wave)), 16, 0, 0);
#pragma unroll
    for (int i = 0; 2 * i + kh < NP; i++)
      __builtin_amdgcn_global_load_lds((const void *)(wsrc[i] + (int64_t)b * BB),
                                       (lds_ptr_t)(w + MX_WROWS * BB * grp + 1024 * (2 * i + kh)),
                                       16, 0, 0);
  };
  f32x16 acc[MS][2];
#pragma unroll
  for (int i = 0; i < MS; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

  // this wave's two chunks of a block from LDS: decode 8 weights per step and
  // tile (w = d*sc*q - dmin*m in fp32, rounded to bf16 nearest-even, as in
  // every matrix-core path) and multiply
  auto multiply_kh = [&](const uint8_t *w, const uint8_t *a, auto khc) {
    constexpr int KH = decltype(khc)::value;
    const uint8_t *wr[2] = {w + BB * (MX_WROWS * grp + n), w + BB * (MX_WROWS * grp + 32 + n)};
    u32x4 hd[2], qh[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
      hd[j] = *(const u32x4 *)wr[j];
      if constexpr (Q5) qh[j] = *(const u32x4 *)(wr[j] + 16 + 16 * h);
    }
#pragma unroll
    for (int cc = 0; cc < 2; cc++) {
      const int c = 2 * KH + cc;
      u32x4 q[2], av[MS][4];
#pragma unroll
      for (int j = 0; j < 2; j++) q[j] = *(const u32x4 *)(wr[j] + QOFF + 32 * c + 16 * h);
#pragma unroll
      for (int i = 0; i < MS; i++)
#pragma unroll
        for (int t = 0; t < 4; t++)
          av[i][t] = *(const u32x4 *)(a + 16 * MX_ASLOTS * (32 * i + n) +
                                      2 * (64 * c + 32 * (t >> 1) + 16 * h + 8 * (t & 1)));
#pragma unroll
      for (int j = 0; j < 2; j++) {
        // Q4_K: a code byte q read as fp8 e4m3 is exactly q * 2^-9 (the small
        // ones as subnormals), so v_cvt_pk_f32_fp8 turns two codes into
        // floats in one instruction and the scale carries 2^9 (exact): the
        // fma forms d*sc*q - dmin*m with the same single rounding as from an
        // integer q. Q5_K codes reach 31, past e4m3's exact integers: one
        // v_cvt_f32_ubyteN per code.
        const RowScales sc = hdr_scales(hd[j], true, c);
#pragma unroll
        for (int t = 0; t < 4; t++) {
          const bool hi = t >= 2;
          const float dm = hi ? sc.b1 : sc.b0;
          uint32_t cw[2];
#pragma unroll
          for (int u = 0; u < 2; u++) {
            const uint32_t d = q[j][2 * (t & 1) + u];
            cw[u] = (hi ? d >> 4 : d) & 0x0F0F0F0Fu;
            if constexpr (Q5) {
              const uint32_t hh = qh[j][2 * (t & 1) + u] >> (2 * c);
              cw[u] |= (hi ? hh << 3 : hh << 4) & 0x10101010u;
            }
          }
          u32x4 bw;
          if constexpr (Q5) {
            const float ds = hi ? sc.a1 : sc.a0;
            bw = u32x4{pack_bf16(ds * (float)(cw[0] & 255u) - dm, ds * (float)((cw[0] >> 8) & 255u) - dm),
                       pack_bf16(ds * (float)((cw[0] >> 16) & 255u) - dm, ds * (float)(cw[0] >> 24) - dm),
                       pack_bf16(ds * (float)(cw[1] & 255u) - dm, ds * (float)((cw[1] >> 8) & 255u) - dm),
                       pack_bf16(ds * (float)((cw[1] >> 16) & 255u) - dm, ds * (float)(cw[1] >> 24) - dm)};
          } else {
            const float ds = (hi ? sc.a1 : sc.a0) * 512.f;
            const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[0], false);
            const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[0], true);
            const auto p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[1], false);
            const auto p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[1], true);
            bw = u32x4{pack_bf16(ds * p0[0] - dm, ds * p0[1] - dm), pack_bf16(ds * p1[0] - dm, ds * p1[1] - dm),
                       pack_bf16(ds * p2[0] - dm, ds * p2[1] - dm), pack_bf16(ds * p3[0] - dm, ds * p3[1] - dm)};
          }
          const bf16x8 bop = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
          for (int i = 0; i < MS; i++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, av[i][t]), bop, acc[i][j], 0, 0, 0);
        }
      }
    }
  };
  auto multiply = [&](const uint8_t *w, const uint8_t *a) {
    if (kh == 0)
      multiply_kh(w, a, std::integral_constant<int, 0>{});
    else
      multiply_kh(w, a, std::integral_constant<int, 1>{});
  };
  __syncthreads();  // every wave is done with buffer 0 (previous pass)
  copy_block(0, sw[0], sa[0]);
  for (int b = 0; b < nbk; b += 2) {
    __syncthreads();  // block b is in buffer 0 for every wave; buffer 1 is free
    if (b + 1 < nbk) copy_block(b + 1, sw[1], sa[1]);
    multiply(sw[0], sa[0]);
    if (b + 1 < nbk) {
      __syncthreads();  // block b+1 is in buffer 1; buffer 0 is free
      if (b + 2 < nbk) copy_block(b + 2, sw[0], sa[0]);
      multiply(sw[1], sa[1]);
    }
  }
  // wave w+4's sums to wave w through the weight buffers, entry tile i in
  // buffer i at [group][j][v][lane] (32 KiB: no copy is in flight and every
  // wave is past its last multiply after the barrier)
  __syncthreads();
  float *xch[MS];
#pragma unroll
  for (int i = 0; i < MS; i++) xch[i] = (float *)sw[i] + grp * 2 * 16 * WAVE + lane;
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < MS; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int v = 0; v < 16; v++) xch[i][(j * 16 + v) * WAVE] = acc[i][j][v];
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int i = 0; i < MS; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] += xch[i][(j * 16 + v) * WAVE];
  // lane holds column n of each 32-column tile and rows 32i + 8(v/4) + 4h + v%4
#pragma unroll
  for (int i = 0; i < MS; i++) {
    const int ent_lane = pent[min(32 * i + n, rows - 1)];
#pragma unroll
    for (int v = 0; v < 16; v++) {
      const int rr = 8 * (v >> 2) + 4 * h + (v & 3);
      const int e_r = __shfl(ent_lane, rr, WAVE);
      if (32 * i + rr < rows) {
        if constexpr (GATEUP) {
          const float g = acc[i][0][v], u = acc[i][1][v];
          const float hv = g / (1.0f + expf(-g)) * u;
          hb[(int64_t)e_r * ldo + col0 + n] = (uint16_t)f32_to_bf16_rne(hv);
        } else {
          float *orow = o + (int64_t)e_r * ldo + col0 + n;
          orow[0] = acc[i][0][v];
          orow[32] = acc[i][1][v];
        }
      }
    }
  }
}

// Grouped matrix-core kernel: workgroup (blockIdx.x, blockIdx.y) = (expert e,
// tile) of eight waves, row group g = wave % 4 with 64 weight rows, over the
// entries perm[offsets[e] ..] of expert e in passes of MX_PASS:
//   GATEUP: A = x rows (token = entry / top_k), K = H; group g's weight tiles
//           are gate rows f0+32g .. f0+32g+31 and up rows F+f0+32g .. of W13[e]
//           (f0 = 128 tile), so g and u of one (entry, f) meet in one lane;
//           hb[entry][f] = bf16 of silu(g) * u.
//   DOWN:   A = hb rows (by entry), K = F; group g's weight tiles are rows
//           r0+64g .. r0+64g+31 and r0+64g+32 .. of W2[e] (r0 = 256 tile);
//           o[entry][r] fp32.
// Consecutive workgroup ids go to different XCDs, so with E a multiple of 8
// the tiles of one expert share an XCD and its L2 holds that expert's A rows.
// Q5 (DOWN only): W2 is Q5_K (176-byte blocks: header, 32-byte high-bit plane,
// 128 code bytes); the decode merges the plane's bits into the codes.
template <bool GATEUP, bool Q5>
__global__ __launch_bounds__(MX_THREADS, 1) void moe_mfma_kernel(
    const uint16_t *__restrict__ a_src, const uint8_t *__restrict__ wq,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm, int top_k, int K,
    int F, int NR, uint16_t *__restrict__ hb, float *__restrict__ o, int H) {
  constexpr int BB = Q5 ? Q5K_BYTES : Q4K_BYTES;
  constexpr int NP = BB / 16;
  // LDS, double-buffered by block: the raw blocks of the 256 weight rows
  // (36,864 B per buffer, Q5_K 45,056 B) and the A rows of a pass (33,792 B
  // per buffer); 141,312 B (Q5_K 157,696 B), one workgroup per compute unit.
  // The buffers are separate variables, so the compiler can tell an LDS read
  // of one buffer from the copy into the other still in flight.
  __shared__ __attribute__((aligned(16))) uint8_t sw0[mx_wbytes(Q5)], sw1[mx_wbytes(Q5)];
  __shared__ __attribute__((aligned(16))) uint8_t sa0[MX_ABYTES], sa1[MX_ABYTES];
  const int e = blockIdx.x, tile = blockIdx.y;
  const int beg = offsets[e], cnt = offsets[e + 1] - beg;
  if (cnt == 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row_bytes = (int64_t)(K / QK) * BB;
  const uint8_t *wexp = wq + (int64_t)e * NR * row_bytes;
  // weight copy sources of this wave: copy 2i + kh of row group grp = wave % 4;
  // its piece p = 64(2i + kh) + lane is piece p % NP of group row p / NP
  // (tile (p / NP) / 32, row (p / NP) % 32 of the tile)
  const int grp = wave & 3, kh = wave >> 2;
  const uint8_t *wsrc[NP / 2 + 1];
#pragma unroll
  for (int i = 0; i < NP / 2 + 1; i++) {
    const int p = min(64 * (2 * i + kh) + lane, 64 * NP - 1), wr = p / NP, j = wr >> 5, nn = wr & 31;
    const int row = GATEUP ? (j == 0 ? 128 * tile + 32 * grp + nn : F + 128 * tile + 32 * grp + nn)
                           : 256 * tile + 64 * grp + 32 * j + nn;
    wsrc[i] = wexp + row * row_bytes + 16 * (p - NP * wr);
  }
  const int ldo = GATEUP ? F : H;
  const int col0 = GATEUP ? 128 * tile + 32 * grp : 256 * tile + 64 * grp;
  uint8_t *const sw[2] = {sw0, sw1}, *const sa[2] = {sa0, sa1};
  for (int p0 = 0; p0 < cnt; p0 += MX_PASS) {
    const int rows = min(MX_PASS, cnt - p0);
    if (rows > 32)
      mx_pass<GATEUP, Q5, 2>(a_src, wsrc, perm + beg + p0, rows, top_k, K, ldo, col0, hb, o, sw, sa);
    else
      mx_pass<GATEUP, Q5, 1>(a_src, wsrc, perm + beg + p0, rows, top_k, K, ldo, col0, hb, o, sw, sa);
  }
}

}  // namespace

// Workspace: a 256-byte status block (word 0: entries of the last call whose
// id was outside [0, E), stored by the routing step of either regime), o
// [n][H] fp32 by entry (both regimes), then h [n][F] fp32 by entry (decode)
// and offsets [E+1], perm [n], hb [n][F] bf16 by entry (matrix cores).
struct MoeWs {
  uint32_t *status;
  float *o, *h;
  int32_t *offsets, *perm;
  uint16_t *hb;
  size_t total;
};

MoeWs carve(void *base, int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F) {
  const int64_t n = T * top_k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return (char *)base + at;
  };
  MoeWs ws;
  ws.status = (uint32_t *)take(256);
  ws.o = (float *)take(sizeof(float) * n * H);
  ws.h = (float *)take(sizeof(float) * n * F);
  ws.offsets = (int32_t *)take(sizeof(int32_t) * (E + 1));
  ws.perm = (int32_t *)take(sizeof(int32_t) * n);
  ws.hb = (uint16_t *)take(sizeof(uint16_t) * n * F);
  ws.total = off;
  return ws;
}

size_t moe_workspace(int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F) {
  return carve(nullptr, T, E, top_k, H, F).total;
}

// Entries processed per pass by the decode kernels, or 0 if the decode regime
// does not apply (too many entries, or inputs too long for LDS). An expert has
// at most T entries when the ids of a token are distinct; passes of
// min(DEC_MT_MAX, T) entries (a power of two) cover a typical expert at once.
int dec_mt(int64_t T, int64_t n, int64_t H, int64_t F, int fr, int rw, size_t &lds1,
           size_t &lds2) {
  if (n > DEC_MAX_N) return 0;
  int start = 1;
  while (start < DEC_MT_MAX && start < T) start <<= 1;
  for (int mt = start; mt >= 1; mt >>= 1) {
    lds1 = (size_t)mt * (H / QK) * REC_BF16 + (size_t)mt * (H / 8) +
           (size_t)mt * 2 * fr * (H / QK) * 4 + (size_t)mt * 2 * fr * 4;
    lds2 = (size_t)mt * (F / QK) * REC_F32 + (size_t)mt * (F / 8) + (size_t)mt * rw * (F / QK) * 4;
    if (lds1 <= 96 * 1024 && lds2 <= 96 * 1024) return mt;
  }
  return 0;
}

// logits != nullptr: the router runs inside the gate+up kernel, which writes
// ids / gw for the two kernels after it.
template <int MT, int FR, int RW, bool Q5>
void launch_dec(const void *x, const void *w13, const void *w2, const int32_t *ids,
                const float *gw, float *y, int64_t T, int64_t E, int64_t top_k, int64_t H,
                int64_t F, const MoeWs &ws, size_t lds1, size_t lds2, hipStream_t s,
                const float *logits) {
  float *hbuf = ws.h, *obuf = ws.o;
  const int n = (int)(T * top_k);
  const unsigned slots = (unsigned)(E < n ? E : n);
  auto k1 = logits ? moe_dec_gateup_kernel<MT, FR, true> : moe_dec_gateup_kernel<MT, FR, false>;
  auto k2 = moe_dec_down_kernel<MT, RW, Q5>;
  (void)hipFuncSetAttribute((const void *)k1, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
  (void)hipFuncSetAttribute((const void *)k2, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
  hipLaunchKernelGGL(k1, dim3((unsigned)((F + FR - 1) / FR), slots), dim3(DEC_THREADS), lds1, s,
                     (const uint16_t *)x, (const uint8_t *)w13, logits ? nullptr : ids, n,
                     (int)top_k, (int)E, (int)H, (int)F, hbuf, logits, (int32_t *)ids,
                     (float *)gw, ws.status);
  hipLaunchKernelGGL(k2, dim3((unsigned)((H + RW - 1) / RW), slots), dim3(DEC_THREADS), lds2, s,
                     hbuf, (const uint8_t *)w2, ids, obuf, n, (int)top_k, (int)E, (int)H, (int)F);
  const int64_t total = T * H / 4;
  hipLaunchKernelGGL(moe_combine_entries_kernel,
                     dim3((unsigned)((total + 255) / 256 < 2048 ? (total + 255) / 256 : 2048)),
                     dim3(256), 0, s, obuf, ids, gw, y, (int)T, (int)top_k, (int)E, (int)H);
}

// Decode regime with tile sizes (FR, RW); false if it does not apply.
template <int FR, int RW, bool Q5>
bool try_dec(const void *x, const void *w13, const void *w2, const int32_t *ids, const float *gw,
             float *y, int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F,
             const MoeWs &ws, hipStream_t s, const float *logits = nullptr) {
  size_t lds1 = 0, lds2 = 0;
  switch (dec_mt(T, T * top_k, H, F, FR, RW, lds1, lds2)) {
    case 4: launch_dec<4, FR, RW, Q5>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, ws, lds1, lds2, s, logits); return true;
    case 2: launch_dec<2, FR, RW, Q5>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, ws, lds1, lds2, s, logits); return true;
    case 1: launch_dec<1, FR, RW, Q5>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, ws, lds1, lds2, s, logits); return true;
    default: return false;
  }
}

// The decode regime with the tile sizes for T tokens; false if it does not apply.
template <bool Q5>
bool try_dec_tiles(const void *x, const void *w13, const void *w2, const int32_t *ids,
                   const float *gw, float *y, int64_t T, int64_t E, int64_t top_k, int64_t H,
                   int64_t F, const MoeWs &ws, hipStream_t s, const float *logits = nullptr) {
  if (T >= DEC_LARGE_FROM_T)
    return try_dec<DEC_FR_LARGE, DEC_RW_LARGE, Q5>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, ws,
                                                   s, logits);
  if (T == 1)
    return try_dec<DEC_FR_ONE, DEC_RW_SMALL, Q5>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, ws, s,
                                                 logits);
  return try_dec<DEC_FR_SMALL, DEC_RW_SMALL, Q5>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, ws, s,
                                                 logits);
}

template <bool Q5>
void launch_moe(const void *x, const void *w13, const void *w2, const int32_t *ids,
                const float *gw, float *y, int64_t T, int64_t E, int64_t top_k, int64_t H,
                int64_t F, void *workspace, hipStream_t s) {
  const int64_t n64 = T * top_k;
  const MoeWs ws = carve(workspace, T, E, top_k, H, F);
  if (try_dec_tiles<Q5>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, ws, s)) return;
  const int n = (int)n64;
  const size_t route_lds = sizeof(int32_t) * E;
  (void)hipFuncSetAttribute((const void *)moe_route_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)route_lds);
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(ROUTE_THREADS), route_lds, s, ids, n,
                     (int)E, ws.offsets, ws.perm, ws.status);
  auto k1 = moe_mfma_kernel<true, false>;
  auto k2 = moe_mfma_kernel<false, Q5>;
  hipLaunchKernelGGL(k1, dim3((unsigned)E, (unsigned)(F / 128)), dim3(MX_THREADS), 0, s,
                     (const uint16_t *)x, (const uint8_t *)w13, ws.offsets, ws.perm, (int)top_k,
                     (int)H, (int)F, (int)(2 * F), ws.hb, (float *)nullptr, (int)H);
  hipLaunchKernelGGL(k2, dim3((unsigned)E, (unsigned)(H / 256)), dim3(MX_THREADS), 0, s,
                     (const uint16_t *)ws.hb, (const uint8_t *)w2, ws.offsets, ws.perm,
                     (int)top_k, (int)F, (int)F, (int)H, (uint16_t *)nullptr, ws.o, (int)H);
  const int64_t total = T * H / 4;
  hipLaunchKernelGGL(moe_combine_entries_kernel,
                     dim3((unsigned)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096)),
                     dim3(256), 0, s, ws.o, ids, gw, y, (int)T, (int)top_k, (int)E, (int)H);
}

void launch_moe_q4k(const void *x, const void *w13, const void *w2, const int32_t *ids,
                    const float *gw, float *y, int64_t T, int64_t E, int64_t top_k, int64_t H,
                    int64_t F, void *workspace, hipStream_t s) {
  launch_moe<false>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, workspace, s);
}

// This device's copy of the scratch array, looked up once per device (with
// that device current) and kept; nullptr if the lookup failed.
void *moe_scratch_ptr() {
  static std::mutex mu;
  static void *ptr[64] = {nullptr};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

void launch_moe_q4k_scratch(const void *x, const void *w13, const void *w2, const int32_t *ids,
                            const float *gw, float *y, int64_t T, int64_t E, int64_t top_k,
                            int64_t H, int64_t F, void *scratch_ptr, hipStream_t s) {
  launch_moe<false>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, scratch_ptr, s);
}

void launch_moe_q4k_q5k(const void *x, const void *w13, const void *w2, const int32_t *ids,
                        const float *gw, float *y, int64_t T, int64_t E, int64_t top_k,
                        int64_t H, int64_t F, void *workspace, hipStream_t s) {
  launch_moe<true>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, workspace, s);
}

void launch_router_topk(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *ids,
                        float *gw, hipStream_t s) {
  constexpr int per_wg = RT_THREADS / WAVE;
  const dim3 grid((unsigned)((T + per_wg - 1) / per_wg)), block(RT_THREADS);
  if (E <= 2 * WAVE)
    hipLaunchKernelGGL(moe_router_topk_kernel<2>, grid, block, 0, s, logits, (int)T, (int)E,
                       (int)k, ids, gw);
  else if (E <= 4 * WAVE)
    hipLaunchKernelGGL(moe_router_topk_kernel<4>, grid, block, 0, s, logits, (int)T, (int)E,
                       (int)k, ids, gw);
  else if (E <= 8 * WAVE)
    hipLaunchKernelGGL(moe_router_topk_kernel<8>, grid, block, 0, s, logits, (int)T, (int)E,
                       (int)k, ids, gw);
  else
    hipLaunchKernelGGL(moe_router_topk_kernel<RT_MAX_E / WAVE>, grid, block, 0, s, logits,
                       (int)T, (int)E, (int)k, ids, gw);
}

// Router then MoE in one call: the ids and gate weights go to the space after
// the MoE workspace.
size_t moe_logits_workspace(int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F) {
  return moe_workspace(T, E, top_k, H, F) + 2 * align256((size_t)(T * top_k) * 4);
}

void launch_moe_from_logits(const void *x, const float *logits, const void *w13, const void *w2,
                            bool down_q5, float *y, int64_t T, int64_t E, int64_t top_k,
                            int64_t H, int64_t F, void *workspace, hipStream_t s) {
  char *extra = (char *)workspace + moe_workspace(T, E, top_k, H, F);
  int32_t *ids = (int32_t *)extra;
  float *gw = (float *)(extra + align256((size_t)(T * top_k) * 4));
  // Decode regime, E <= 128 and at most one token per wave of the gate+up
  // kernel: the router runs inside that kernel (T = 1: 26.8 -> 25.1 us). With
  // more tokens a wave routes several in turn before any weight is read,
  // which cost more than the separate router launch (T = 8: 65 -> 70 us).
  if (E <= 2 * WAVE && T <= DEC_THREADS / WAVE) {
    const MoeWs ws = carve(workspace, T, E, top_k, H, F);
    const bool done =
        down_q5 ? try_dec_tiles<true>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, ws, s, logits)
                : try_dec_tiles<false>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, ws, s, logits);
    if (done) return;
  }
  launch_router_topk(logits, T, E, top_k, ids, gw, s);
  if (down_q5)
    launch_moe<true>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, workspace, s);
  else
    launch_moe<false>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, workspace, s);
}

}  // namespace qdm
